"""Parity comparator between a candidate result and the oracle.  TEST INFRASTRUCTURE ONLY.

fp64 rule (near-tie reading): codes must be equal, except at an entry whose
oracle pre-rounding value y = x/s lies within ``tie_tol`` grid units of a
rounding boundary (|frac(y) - 1/2| < tie_tol).  At such an entry the oracle is
re-run with the candidate's code imposed there and the comparison continues
downstream (equal-up-to-ties is the only sense in which floating-point runs of
different summation orders can agree, as the BaKron review notes for the
equivalence theorem).

fp32 rule: the fraction of differing codes and the relative difference of the
proxy loss are reported and compared against the caller's bounds.
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


def mismatch_fraction(Z_a, Z_b) -> float:
    return float(np.mean(np.asarray(Z_a) != np.asarray(Z_b)))


def rel_diff(a: float, b: float) -> float:
    return abs(a - b) / max(abs(b), 1e-300)
