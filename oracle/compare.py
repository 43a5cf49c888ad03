"""Parity comparator between a candidate result and the oracle.  TEST INFRASTRUCTURE ONLY.

fp64 rule (near-tie reading): codes must be equal, except at an entry whose
oracle pre-rounding value y = x/s lies within ``tie_tol`` grid units of a
rounding boundary (|frac(y) - 1/2| < tie_tol).  At such an entry the oracle is
re-run with the candidate's code imposed there and the comparison continues
downstream (equal-up-to-ties is the only sense in which floating-point runs of
different summation orders can agree, as the BaKron review notes for the
equivalence theorem).

fp32 rule: the fraction of differing codes and the relative difference of the
proxy loss are reported and compared against the caller's bounds.  In single
precision one near-tie decision that goes the other way changes every later
entry it feeds (the oracle's own fp32 loop differs from its fp64 loop on a few
percent of a 4096 x 4096 layer that way), so large fp32 runs are also checked
along their own trajectory: the oracle is run with every code imposed from the
candidate, which gives the exact pre-rounding values that the candidate's
earlier decisions imply, and each candidate code must be the rounding of its
value except where that value lies within ``tie_tol`` of a boundary.
"""
from __future__ import annotations

import numpy as np

from . import o3

NOT_FORCED = o3.NOT_FORCED


def tie_distance(Y: np.ndarray) -> np.ndarray:
    """|frac(y) - 1/2|: distance of the pre-rounding value from a rounding boundary."""
    return np.abs(Y - np.floor(Y) - 0.5)


def first_in_antidiagonal_order(mask: np.ndarray):
    idx = np.argwhere(mask)
    if idx.size == 0:
        return None
    key = idx[:, 0] + idx[:, 1]
    best = np.lexsort((idx[:, 0], key))[0]
    return tuple(idx[best])


def codes_equal_up_to_ties(Z_cand, run_oracle, tie_tol=1e-9, max_forced=64):
    """run_oracle(force) -> (Z, Y).  Returns (ok, n_forced, info)."""
    Z_cand = np.asarray(Z_cand).astype(np.int32)
    force = None
    n_forced = 0
    while True:
        Z, Y = run_oracle(force)
        bad = np.asarray(Z).astype(np.int32) != Z_cand
        first = first_in_antidiagonal_order(bad)
        if first is None:
            return True, n_forced, "equal"
        i, j = int(first[0]), int(first[1])
        if tie_distance(Y[i, j]) >= tie_tol:
            return False, n_forced, (f"code mismatch at ({i}, {j}): candidate {int(Z_cand[i, j])} oracle "
                                     f"{int(Z[i, j])}, y={float(Y[i, j])!r}, {int(bad.sum())} mismatches")
        if n_forced >= max_forced:
            return False, n_forced, "too many near-tie entries"
        if force is None:
            force = np.full(Z_cand.shape, NOT_FORCED, np.int32)
        force[i, j] = Z_cand[i, j]
        n_forced += 1


def trajectory_violations(Z_cand, Y_forced, bits, tie_tol):
    """Entries where the candidate's code is not clamp(rne(y)) of the pre-rounding
    value y that the oracle computed with every code imposed from the candidate.

    Returns (violations, near_ties): violations are such entries with y farther
    than ``tie_tol`` from a rounding boundary; near_ties are the ones within it.
    Non-finite y (a zero scale) expects code 0.  bits=None: unbounded codes.
    """
    qmin, qmax = (-np.inf, np.inf) if bits is None else (-(1 << (bits - 1)), (1 << (bits - 1)) - 1)
    Y = np.asarray(Y_forced, dtype=np.float64)
    finite = np.isfinite(Y)
    own = np.where(finite, np.clip(np.rint(np.where(finite, Y, 0.0)), qmin, qmax), 0.0)
    differ = own != np.asarray(Z_cand).astype(np.float64)
    near = differ & finite & (tie_distance(np.where(finite, Y, 0.0)) < tie_tol)
    return int((differ & ~near).sum()), int(near.sum())


def mismatch_roots(mask) -> np.ndarray:
    """The differing entries that no other differing entry precedes.

    An entry's pre-rounding value depends only on the codes to its top-left
    (componentwise <=, FastKron page section 2.3), so where two runs first part
    ways every later difference lies in the bottom-right cone of an earlier one.
    A root is a difference with no other difference in its top-left rectangle:
    every code it depends on is equal in both runs, so both saw the same exact
    pre-rounding value there and the split can only be a near-tie decision.
    """
    M = np.asarray(mask, dtype=bool)
    P = np.logical_or.accumulate(np.logical_or.accumulate(M, axis=0), axis=1)
    above = np.zeros_like(M)
    above[1:, :] = P[:-1, :]
    left = np.zeros_like(M)
    left[:, 1:] = P[:, :-1]
    return M & ~above & ~left


def mismatch_fraction(Z_a, Z_b) -> float:
    return float(np.mean(np.asarray(Z_a) != np.asarray(Z_b)))


def rel_diff(a: float, b: float) -> float:
    return abs(a - b) / max(abs(b), 1e-300)
