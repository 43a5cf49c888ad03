"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: the
printed Kronecker example, exact rational agreement of every processing order
(FastKron page section 2.5's equivalence theorem), closed forms, textbook special
cases (one-sided GPTQ, round-to-nearest) and structural properties (the
bottom-right update of section 2.3).  The mutation tests at the end plant
plausible mistakes in oracle copies and check that the pins catch them.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import synth
from oracle import compare, dense, exact, o3
from tests.conftest import read_golden


def _factors(prob, delta=0.01):
    A = dense.factor_accumulate(prob["act"], alpha=1.0 / prob["act"].shape[0])
    B = dense.factor_accumulate(prob["grad"], alpha=1.0 / prob["grad"].shape[0])
    Ad, UA = dense.prepare(A, delta)
    Bd, UB = dense.prepare(B, delta)
    return Ad, UA, Bd, UB


@pytest.fixture(scope="module")
def tiny():
    c = synth.tiny()
    Ad, UA, Bd, UB = _factors(c)
    s = dense.scales(c["W"], 4, False)
    return c, Ad, UA, Bd, UB, s


# ---------------------------------------------------------------- conventions

def test_kron_convention_matches_printed_example():
    g = read_golden("kronq_kron_example.txt")
    P = g["PRINTED_KRON"]
    # every 2x2 block is a multiple of the same matrix: the first factor indexes blocks
    G = P[:2, :2] / P[0, 0] * g["READING_H_G"][0, 0]
    for a in range(2):
        for b in range(2):
            blk = P[2 * a:2 * a + 2, 2 * b:2 * b + 2]
            assert np.allclose(blk, g["READING_H_X"][a, b] * g["READING_H_G"])
    assert np.array_equal(np.kron(g["READING_H_X"], g["READING_H_G"]), P)
    assert np.allclose(G, g["READING_H_G"])


def test_kron_acts_on_column_major_vec():
    # (A (x) B) vecop(E) = vecop(B E A^T): the Hessian of tr(B E A E^T) in vecop
    # coordinates is A (x) B only with column-major vectorisation.
    r = np.random.default_rng(0)
    m, n = 3, 4
    A = r.standard_normal((n, n)); A = A @ A.T
    B = r.standard_normal((m, m)); B = B @ B.T
    E = r.standard_normal((m, n))
    e = E.reshape(-1, order="F")
    assert np.allclose(np.kron(A, B) @ e, (B @ E @ A.T).reshape(-1, order="F"))
    assert np.isclose(e @ np.kron(A, B) @ e, np.trace(B @ E @ A @ E.T))


def test_hat_factor_is_kron_of_factors(tiny):
    c, Ad, UA, Bd, UB, s = tiny
    _, _, _, Uh = dense.vectorized_kron_gptq(c["W"], Ad, Bd, s, 4, return_factor=True)
    assert np.max(np.abs(Uh - np.kron(UA, UB))) < 1e-12


def test_prepare_routes_agree_and_invert():
    c = synth.spectral(64, 48)
    for M in (c["A"], c["B"]):
        Md = dense.damp(M, 0.01)
        U1 = dense.upper_factor_via_inverse(Md)
        U2 = dense.upper_factor_via_reverse_cholesky(Md)
        assert np.allclose(np.tril(U1, -1), 0) and np.all(np.diag(U1) > 0)
        assert np.max(np.abs(U1.T @ U1 @ Md - np.eye(len(M)))) < 1e-9
        assert np.max(np.abs(U1 - U2)) < 1e-9 * np.max(np.abs(U1))


def test_damp_is_relative_to_mean_diagonal():
    A = np.diag([1.0, 2.0, 3.0, 6.0])
    assert np.array_equal(dense.damp(A, 0.5) - A, 1.5 * np.eye(4))


def test_factor_accumulate_brute_force_and_closed_form():
    r = np.random.default_rng(1)
    X = r.standard_normal((7, 5))
    S0 = r.standard_normal((5, 5))
    want = 0.5 * S0
    for row in X:
        want = want + 0.25 * np.outer(row, row)
    assert np.allclose(dense.factor_accumulate(X, S0, 0.25, 0.5), want, atol=1e-13)
    q, _ = np.linalg.qr(r.standard_normal((9, 4)))
    sig = np.array([1.0, 2.0, 3.0, 4.0])
    G = dense.factor_accumulate(q * sig, alpha=1.0)
    assert np.allclose(G, np.diag(sig ** 2), atol=1e-13)


def test_scales_definition():
    W = np.array([[1.0, -7.0, 2.0], [0.5, 0.25, -0.125]])
    assert np.array_equal(dense.scales(W, 4, True), np.array([1.0, 0.5 / 7]))
    assert np.array_equal(dense.scales(W, 4, False), np.array([1.0]))
    assert np.array_equal(dense.scales(W, 2, True), np.array([7.0, 0.5]))
    assert dense.grid(2) == (-2, 1) and dense.grid(3) == (-4, 3) and dense.grid(4) == (-8, 7)


def test_quantizer_round_half_even_and_clamp():
    assert dense.quantize(2.5, 1.0, -8, 7)[0] == 2
    assert dense.quantize(3.5, 1.0, -8, 7)[0] == 4
    assert dense.quantize(-2.5, 1.0, -8, 7)[0] == -2
    assert dense.quantize(9.0, 1.0, -8, 7)[0] == 7
    assert dense.quantize(-20.0, 2.0, -8, 7)[0] == -8
    assert dense.quantize(1.0, 0.0, -8, 7)[:2] == (0.0, 0.0)
    assert exact.rne(Fr(5, 2)) == 2 and exact.rne(Fr(7, 2)) == 4 and exact.rne(Fr(-5, 2)) == -2
    assert exact.rne(Fr(-7, 3)) == -2 and exact.rne(Fr(8, 3)) == 3


# ------------------------------------------------- exact equivalence (tier O0)

EXACT_CASES = [(3, 4, 3, 11), (4, 3, 2, 12), (4, 4, 4, 13), (1, 5, 3, 14), (5, 1, 3, 15),
               (2, 6, 2, 16), (6, 6, 3, 17)]


def _exact_problem(m, n, bits, seed, unit_step=False):
    p = synth.small_integer_problem(seed, m, n)
    W = exact.to_fr(p["W"])
    A = exact.matmul(exact.transpose(exact.to_fr(p["act"])), exact.to_fr(p["act"]))
    B = exact.matmul(exact.transpose(exact.to_fr(p["grad"])), exact.to_fr(p["grad"]))
    Ad, Bd = exact.damp(A, Fr(1, 100)), exact.damp(B, Fr(1, 100))
    NA, uA = exact.normalized_factor(Ad)
    NB, uB = exact.normalized_factor(Bd)
    qmax = (1 << (bits - 1)) - 1
    if unit_step:
        s = [Fr(1)] * m
    else:
        s = [max(abs(x) for x in row) / qmax or Fr(1) for row in W]
    return dict(W=W, Ad=Ad, Bd=Bd, NA=NA, NB=NB, uA=uA, uB=uB, s=s, bits=bits, raw=p)


@pytest.mark.parametrize("m,n,bits,seed", EXACT_CASES)
def test_exact_all_orders_identical(m, n, bits, seed):
    P = _exact_problem(m, n, bits, seed)
    args = (P["W"], P["NA"], P["NB"], P["s"], bits)
    ref = exact.naive(*args, order="column")
    runs = [exact.naive(*args, order="row"), exact.naive(*args, order="antidiagonal"),
            exact.left_looking(*args), exact.recursive(*args, over="antidiagonal"),
            exact.recursive(*args, over="vecop")]
    for Z, D in runs:
        assert Z == ref[0] and D == ref[1]


@pytest.mark.parametrize("m,n,bits,seed", EXACT_CASES[:4])
def test_exact_loss_identity(m, n, bits, seed):
    # V - W = L~_B Delta L~_A^T  =>  tr(B E A E^T) = sum Delta_ij^2 / (U_B,ii^2 U_A,jj^2)
    P = _exact_problem(m, n, bits, seed)
    Z, D = exact.naive(P["W"], P["NA"], P["NB"], P["s"], bits)
    V = [[P["s"][i] * Z[i][j] for j in range(n)] for i in range(m)]
    closed = sum(D[i][j] ** 2 / (P["uB"][i] * P["uA"][j]) for i in range(m) for j in range(n))
    assert exact.loss(P["W"], V, P["Ad"], P["Bd"]) == closed


@pytest.mark.parametrize("m,n,seed", [(3, 4, 21), (5, 5, 22), (2, 6, 23)])
def test_exact_error_bound_unit_step(m, n, seed):
    # Unclipped unit grid: loss <= 1/4 tr(A_d) tr(B_d) (BaKron review, forward_implications[4]).
    P = _exact_problem(m, n, 16, seed, unit_step=True)
    Z, D = exact.naive(P["W"], P["NA"], P["NB"], P["s"], 16)
    assert all(abs(d) <= Fr(1, 2) for row in D for d in row)
    V = [[Fr(Z[i][j]) for j in range(n)] for i in range(m)]
    trA = sum(P["Ad"][i][i] for i in range(n))
    trB = sum(P["Bd"][i][i] for i in range(m))
    assert exact.loss(P["W"], V, P["Ad"], P["Bd"]) <= Fr(1, 4) * trA * trB


@pytest.mark.parametrize("m,n,bits,seed", EXACT_CASES)
def test_float_tiers_match_exact(m, n, bits, seed):
    P = _exact_problem(m, n, bits, seed)
    Zx, _ = exact.naive(P["W"], P["NA"], P["NB"], P["s"], bits)
    raw = P["raw"]
    A = raw["act"].T @ raw["act"] * 1.0
    B = raw["grad"].T @ raw["grad"] * 1.0
    Ad, UA = dense.prepare(A, 0.01)
    Bd, UB = dense.prepare(B, 0.01)
    s = np.array([float(x) for x in P["s"]])
    W = raw["W"].astype(np.float64)
    Zx = np.array(Zx)
    Z1, _, Y1 = dense.vectorized_kron_gptq(W, Ad, Bd, s, bits)
    Z2, _, Y2, _ = dense.two_sided_naive(W, UA, UB, s, bits, "antidiagonal")
    Z3, _, Y3, _ = o3.solve(W, UA, UB, s, bits)
    for Z, Y in ((Z1, Y1), (Z2, Y2), (Z3, Y3)):
        near = compare.tie_distance(Y) < 1e-9
        assert np.all((Z == Zx) | near)


# ------------------------------------------------------- floating-point tiers

def test_o1_o2_o3_recursive_identical_on_tiny(tiny):
    c, Ad, UA, Bd, UB, s = tiny
    Z1, V1, Y1 = dense.vectorized_kron_gptq(c["W"], Ad, Bd, s, 4)
    assert compare.tie_distance(Y1).min() > 1e-9
    for order in ("column", "row", "antidiagonal"):
        Z2, V2, _, _ = dense.two_sided_naive(c["W"], UA, UB, s, 4, order)
        assert np.array_equal(Z1, Z2) and np.array_equal(V1, V2)
    Zr, _, _, _ = dense.two_sided_recursive(c["W"], UA, UB, s, 4)
    Zv, _, _, _ = dense.two_sided_recursive_vecop(c["W"], UA, UB, s, 4)
    Z3, V3, _, D3 = o3.solve(c["W"], UA, UB, s, 4)
    assert np.array_equal(Z1, Zr) and np.array_equal(Z1, Zv) and np.array_equal(Z1, Z3)
    loss = dense.proxy_loss(c["W"], V3, Ad, Bd)
    assert abs(loss - dense.loss_from_errors(D3, UA, UB)) < 1e-12 * loss


def test_b_identity_is_one_sided_gptq():
    c = synth.spectral(64, 48, config=2)
    Ad, UA = dense.prepare(c["A"], 0.01)
    s = dense.scales(c["W"], 3, True)
    Zg, Vg = dense.one_sided_gptq(c["W"], UA, s, 3)
    Zn, Vn, _, _ = dense.two_sided_naive(c["W"], UA, np.eye(64), s, 3)
    Z3, V3, _, _ = o3.solve(c["W"], UA, None, s, 3)
    Z3b, V3b, _, _ = o3.solve(c["W"], UA, np.eye(64), s, 3)
    for Z, V in ((Zn, Vn), (Z3, V3), (Z3b, V3b)):
        assert np.array_equal(Z, Zg) and np.array_equal(V, Vg)


def test_identity_factors_is_round_to_nearest():
    c = synth.spectral(40, 30, config=2)
    s = dense.scales(c["W"], 3, True)
    Z, V, _, _ = o3.solve(c["W"], np.eye(30), np.eye(40), s, 3)
    want = np.clip(np.rint(c["W"] / s[:, None]), -4, 3)
    assert np.array_equal(Z, want) and np.array_equal(V, want * s[:, None])


def test_single_row_and_single_column():
    c = synth.spectral(24, 20, config=2)
    AdA, UA = dense.prepare(c["A"][:20, :20], 0.01)
    BdB, UB = dense.prepare(c["B"][:24, :24], 0.01)
    # m = 1: GPTQ along the row with A
    w = c["W"][:1, :]
    s = dense.scales(w, 3, False)
    Z, _, _, _ = o3.solve(w, UA, np.ones((1, 1)), s, 3)
    Zg, _ = dense.one_sided_gptq(w, UA, s, 3)
    assert np.array_equal(Z, Zg)
    # n = 1: GPTQ down the column with B (per-tensor scale)
    w = c["W"][:, :1]
    s = dense.scales(w, 3, False)
    Z, _, _, _ = o3.solve(w, np.ones((1, 1)), UB, s, 3)
    Zg, _ = dense.one_sided_gptq(w.T, UB, s, 3)
    assert np.array_equal(Z, Zg.T)


def test_prefix_property():
    # The top-left k x k corner depends only on the corners of W, U_A, U_B and s
    # (updates only move to the bottom-right, FastKron page section 2.3).
    c = synth.spectral(96, 80, config=2)
    Ad, UA = dense.prepare(c["A"], 0.01)
    Bd, UB = dense.prepare(c["B"], 0.01)
    s = dense.scales(c["W"], 3, True)
    Z, V, _, _ = o3.solve(c["W"], UA, UB, s, 3)
    for k in (1, 17, 48):
        Zk, Vk, _, _ = o3.solve(c["W"][:k, :k], UA[:k, :k], UB[:k, :k], s[:k], 3)
        assert np.array_equal(Zk, Z[:k, :k]) and np.array_equal(Vk, V[:k, :k])
    Zr, _, _, _ = o3.solve(c["W"][:30, :], UA, UB[:30, :30], s[:30], 3)
    assert np.array_equal(Zr, Z[:30, :])


def test_transpose_symmetry_per_tensor_scale():
    c = synth.spectral(40, 56, config=2)
    Ad, UA = dense.prepare(c["A"][:56, :56], 0.01)
    Bd, UB = dense.prepare(c["B"][:40, :40], 0.01)
    s = dense.scales(c["W"], 3, False)
    Z, _, _, _ = o3.solve(c["W"], UA, UB, s, 3)
    Zt, _, _, _ = o3.solve(c["W"].T, UB, UA, s, 3)
    assert np.array_equal(Z, Zt.T)


def test_scale_invariance_of_factors():
    c = synth.spectral(32, 32, config=2)
    _, U1 = dense.prepare(c["A"], 0.01)
    _, U4 = dense.prepare(4.0 * c["A"], 0.01)
    assert np.array_equal(dense.normalized_factor(U1), dense.normalized_factor(U4))


def test_o3_matches_o2_on_spectral_256():
    c = synth.spectral()
    Ad, UA = dense.prepare(c["A"], 0.01)
    Bd, UB = dense.prepare(c["B"], 0.01)
    s = dense.scales(c["W"], 3, True)
    Z2, V2, Y2, D2 = dense.two_sided_naive(c["W"], UA, UB, s, 3, "antidiagonal")
    Z3, V3, Y3, D3 = o3.solve(c["W"], UA, UB, s, 3)
    assert compare.tie_distance(Y3).min() > 1e-9
    assert np.array_equal(Z2, Z3)
    l2 = dense.proxy_loss(c["W"], V2, Ad, Bd)
    assert abs(l2 - dense.loss_from_errors(D3, UA, UB)) < 1e-11 * l2


def test_o3_fp32_floor_spectral_256():
    c = synth.spectral()
    Ad, UA = dense.prepare(c["A"], 0.01)
    Bd, UB = dense.prepare(c["B"], 0.01)
    s = dense.scales(c["W"], 3, True)
    Z64, V64, _, _ = o3.solve(c["W"], UA, UB, s, 3)
    Z32, V32, _, _ = o3.solve(c["W"], UA, UB, s, 3, dtype=np.float32)
    assert compare.mismatch_fraction(Z32, Z64) <= 1e-3
    l64 = dense.proxy_loss(c["W"], V64, Ad, Bd)
    l32 = dense.proxy_loss(c["W"], V32.astype(np.float64), Ad, Bd)
    assert compare.rel_diff(l32, l64) <= 1e-3


# --------------------------------------------------------------- comparator

def test_comparator_accepts_forced_tie_and_rejects_real_mismatch():
    c = synth.spectral(20, 16, config=2)
    Ad, UA = dense.prepare(c["A"][:16, :16], 0.01)
    Bd, UB = dense.prepare(c["B"][:20, :20], 0.01)
    W = c["W"].copy()
    s = np.full(20, 0.25)
    W[0, 0] = 2.5 * 0.25  # an exact tie at the first entry: rne gives 2
    run = lambda f: o3.solve(W, UA, UB, s, 3, force=f)[0::2]
    Z, Y = run(None)
    assert Z[0, 0] == 2 and compare.tie_distance(Y[0, 0]) == 0.0
    force = np.full(W.shape, compare.NOT_FORCED, np.int32)
    force[0, 0] = 3
    Zalt = o3.solve(W, UA, UB, s, 3, force=force)[0]
    assert not np.array_equal(Zalt, Z)
    ok, nf, _ = compare.codes_equal_up_to_ties(Zalt, run)
    assert ok and nf == 1
    bad = Z.copy()
    bad[5, 7] = bad[5, 7] + 1 if bad[5, 7] < 3 else bad[5, 7] - 1
    ok, _, info = compare.codes_equal_up_to_ties(bad, run)
    assert not ok and "(5, 7)" in info


def test_trajectory_check_accepts_near_tie_branch_and_rejects_wrong_code():
    # A candidate that took the other branch at one near-tie entry, and followed
    # its own trajectory afterwards, is valid; a code changed anywhere else is not.
    c = synth.spectral()
    _, UA = dense.prepare(c["A"], 0.01)
    _, UB = dense.prepare(c["B"], 0.01)
    s = dense.scales(c["W"], 3, True)
    Z, _, Y, _ = o3.solve(c["W"], UA, UB, s, 3)
    Yf = o3.solve(c["W"], UA, UB, s, 3, force=Z.astype(np.int32))[2]
    assert compare.trajectory_violations(Z, Yf, 3, 1e-4) == (0, 0)
    td = compare.tie_distance(Y)
    i, j = np.unravel_index(np.argmin(np.where(np.abs(Y) < 3.0, td, 1.0)), Y.shape)
    force = np.full(Z.shape, compare.NOT_FORCED, np.int32)
    force[i, j] = Z[i, j] + (1 if Y[i, j] > Z[i, j] else -1)  # the other side of the boundary
    Zb = o3.solve(c["W"], UA, UB, s, 3, force=force)[0]
    Yb = o3.solve(c["W"], UA, UB, s, 3, force=Zb.astype(np.int32))[2]
    viol, near = compare.trajectory_violations(Zb, Yb, 3, max(2 * td[i, j], 1e-12))
    assert viol == 0 and near == 1
    bad = Z.copy()
    k = np.unravel_index(np.argmax(np.where(Z == 0, td, -1.0)), Z.shape)  # far from a boundary
    bad[k] = 1
    Ybad = o3.solve(c["W"], UA, UB, s, 3, force=bad.astype(np.int32))[2]
    viol, _ = compare.trajectory_violations(bad, Ybad, 3, 1e-4)
    assert viol >= 1


def test_mismatch_roots_are_the_minimal_differences():
    M = np.zeros((6, 7), bool)
    M[1, 4] = M[3, 2] = True          # two roots: neither precedes the other
    M[2, 5] = M[4, 4] = M[5, 6] = True  # inside the cones of the roots
    M[0, 6] = True                     # a root far to the right
    R = compare.mismatch_roots(M)
    assert sorted(zip(*np.nonzero(R))) == [(0, 6), (1, 4), (3, 2)]
    # brute force: a difference is a root iff no other difference is <= it componentwise
    r = np.random.default_rng(3)
    for _ in range(20):
        M = r.random((9, 8)) < 0.08
        want = np.zeros_like(M)
        for i, j in zip(*np.nonzero(M)):
            want[i, j] = not any(M[a, b] and (a, b) != (i, j) for a in range(i + 1) for b in range(j + 1))
        assert np.array_equal(compare.mismatch_roots(M), want)


def test_first_branch_of_a_forced_run_is_its_only_root():
    # Forcing one code away from the oracle's changes only that entry's bottom-right cone.
    c = synth.spectral(40, 30, config=2)
    _, UA = dense.prepare(c["A"][:30, :30], 0.01)
    _, UB = dense.prepare(c["B"][:40, :40], 0.01)
    s = dense.scales(c["W"], 3, True)
    Z = o3.solve(c["W"], UA, UB, s, 3)[0]
    force = np.full(Z.shape, compare.NOT_FORCED, np.int32)
    force[7, 9] = Z[7, 9] + (1 if Z[7, 9] < 3 else -1)
    Zf = o3.solve(c["W"], UA, UB, s, 3, force=force)[0]
    diff = Zf != Z
    assert diff.sum() > 1 and not diff[:7, :].any() and not diff[:, :9].any()
    assert sorted(zip(*np.nonzero(compare.mismatch_roots(diff)))) == [(7, 9)]


def test_sensitivity_is_the_trace_of_the_kronecker_factor():
    # KronQ page: the score of a sublayer is tr(H_X) tr(H_G).  For the printed
    # 4x4 example H_X (x) H_G its trace is 8 + 10 + 12 + 15 = 45 = tr(H_X) tr(H_G).
    g = read_golden("kronq_kron_example.txt")
    P = g["PRINTED_KRON"]
    assert dense.sensitivity(g["READING_H_X"], g["READING_H_G"]) == 45.0 == np.trace(P)
    assert dense.sensitivity(np.diag([1.0, 2.0, 3.0]), np.diag([4.0, 5.0])) == 54.0
    # the score uses the undamped factors; uniform relative damping delta would
    # scale every score by (1 + delta)^2 and leave the ranking unchanged
    r = np.random.default_rng(5)
    A = r.standard_normal((6, 6)); A = A @ A.T
    B = r.standard_normal((4, 4)); B = B @ B.T
    sd = dense.sensitivity(dense.damp(A, 0.01), dense.damp(B, 0.01))
    assert abs(sd - 1.01 ** 2 * dense.sensitivity(A, B)) <= 1e-12 * sd


# ------------------------------------------------------------ mutation tests

def test_pins_catch_planted_mistakes(tiny):
    c, Ad, UA, Bd, UB, s = tiny
    Z1, _, _ = dense.vectorized_kron_gptq(c["W"], Ad, Bd, s, 4)
    # transposed operand: factors swapped between the two sides
    Zs, _, _, _ = o3.solve(c["W"], UB, UA, s, 4)
    assert not np.array_equal(Zs, Z1)
    # dropped column feedback: B ignored
    Zd, _, _, _ = o3.solve(c["W"], UA, None, s, 4)
    assert not np.array_equal(Zd, Z1)
    # wrong sign of the feedback: use -L~ off the diagonal (i.e. U with negated rows)
    UAneg = 2 * np.diag(np.diag(UA)) - UA
    Zn, _, _, _ = o3.solve(c["W"], UAneg, UB, s, 4)
    assert not np.array_equal(Zn, Z1)
    # Kronecker order swapped in the literal tier
    Zk, _, _ = dense.vectorized_kron_gptq(c["W"].T.copy(), Ad, Bd, s, 4)
    assert not np.array_equal(Zk.T, Z1)


# ------------------------------------------------ WaterKron rate allocation

def test_waterkron_scales_are_reverse_cholesky_reciprocals():
    # WaterKron page section 3: alpha_j proportional to 1 / L_jj with L the reverse
    # Cholesky factor (L^T L = A).  By hand for A = [[10, 2], [2, 4]]: L = [[3, 0],
    # [1, 2]], so alpha = step * (1/3, 1/2); B = I gives beta = 1 (WaterSIC).
    A = np.array([[10.0, 2.0], [2.0, 4.0]])
    L = np.array([[3.0, 0.0], [1.0, 2.0]])
    assert np.allclose(L.T @ L, A)
    UA = dense.upper_factor_via_reverse_cholesky(A)
    alpha, beta = dense.waterkron_scales(UA, None, 0.5, m=3)
    assert np.allclose(alpha, [0.5 / 3, 0.25], rtol=1e-14) and np.array_equal(beta, np.ones(3))
    B = np.array([[4.0, 0.0], [0.0, 9.0]])
    _, beta = dense.waterkron_scales(UA, dense.upper_factor_via_inverse(B), 1.0)
    assert np.allclose(beta, [0.5, 1.0 / 3.0], rtol=1e-14)


def test_empirical_entropy_definition():
    assert dense.empirical_entropy([0, 0, 1, 1]) == 1.0
    assert dense.empirical_entropy(np.arange(8)) == 3.0
    assert dense.empirical_entropy(np.full((4, 4), 7)) == 0.0
    assert abs(dense.empirical_entropy([0, 0, 0, 1]) - (2 - 0.75 * np.log2(3))) < 1e-15


@pytest.fixture(scope="module")
def waterkron_tiny(tiny):
    c, Ad, UA, Bd, UB, s = tiny
    step = 0.05
    alpha, beta = dense.waterkron_scales(UA, UB, step)
    return c, Ad, UA, Bd, UB, alpha, beta


def test_waterkron_tiers_agree(waterkron_tiny):
    # Per-entry steps beta_i alpha_j and unbounded codes: the literal Kronecker
    # GPTQ (with the vectorised scale alpha (x) beta), the matrix loop in two
    # orders and the left-looking loop give the same codes.
    c, Ad, UA, Bd, UB, alpha, beta = waterkron_tiny
    Z1, V1, Y1 = dense.vectorized_kron_gptq(c["W"], Ad, Bd, beta, None, alpha=alpha)
    assert compare.tie_distance(Y1).min() > 1e-9
    Z2c, _, _, _ = dense.two_sided_naive(c["W"], UA, UB, beta, None, "column", alpha=alpha)
    Z2a, _, _, _ = dense.two_sided_naive(c["W"], UA, UB, beta, None, "antidiagonal", alpha=alpha)
    Z3, V3, _, D3 = o3.solve(c["W"], UA, UB, beta, None, alpha=alpha)
    assert Z3.dtype == np.int32
    for Z in (Z2c, Z2a, Z3):
        assert np.array_equal(Z, Z1)
    assert np.max(np.abs(Z1)) > 8  # beyond a 4-bit grid: the codes are not clipped
    assert np.allclose(V3, V1, rtol=0, atol=1e-12)
    l1 = dense.proxy_loss(c["W"], V1, Ad, Bd)
    assert abs(l1 - dense.loss_from_errors(D3, UA, UB)) <= 1e-11 * l1


def test_watersic_is_one_sided_gptq_with_column_scales():
    c = synth.spectral(48, 40, config=2)
    _, UA = dense.prepare(c["A"][:40, :40], 0.01)
    alpha, beta = dense.waterkron_scales(UA, None, 0.02, m=48)
    Zr, Vr = dense.one_sided_gptq(c["W"], UA, beta, None, alpha=alpha)
    Z3, V3, Y3, _ = o3.solve(c["W"], UA, None, beta, None, alpha=alpha)
    assert compare.tie_distance(Y3).min() > 1e-9
    assert np.array_equal(Z3, Zr) and np.allclose(V3, Vr, rtol=0, atol=1e-12)


def test_waterkron_high_rate_distortion_is_uniform():
    # With alpha_j beta_i = step U_A,jj U_B,ii every rounding error, measured in
    # the loss geometry (Delta_ij / (U_B,ii U_A,jj)), is step times a value in
    # [-1/2, 1/2]; at a fine step these are uniform, so the proxy loss is
    # m n step^2 / 12 (the high-rate regime of the WaterKron page, appendix C.2).
    c = synth.spectral(64, 64, config=2)
    Ad, UA = dense.prepare(c["A"], 0.01)
    Bd, UB = dense.prepare(c["B"], 0.01)
    # a step a thousandth of the weights' spread in the transformed geometry
    step = 1e-3 * np.sqrt(np.mean((c["W"] / np.outer(np.diag(UB), np.diag(UA))) ** 2))
    alpha, beta = dense.waterkron_scales(UA, UB, step)
    Z, V, _, D = o3.solve(c["W"], UA, UB, beta, None, alpha=alpha)
    S = np.outer(beta, alpha)
    assert np.max(np.abs(D / S)) <= 0.5 + 1e-9
    assert np.max(np.abs(Z)) > 127  # far beyond an 8-bit grid
    loss = dense.proxy_loss(c["W"], V, Ad, Bd)
    ratio = loss / (64 * 64 * step ** 2 / 12)
    assert abs(ratio - 1.0) < 0.05, ratio


# ------------------------------------- Kronecker approximations (FlipFlop, Frobenius)

def _paired_samples(seed, N, n, m):
    r = synth.rng(seed)
    Xa = r.standard_normal((N, n)) * np.exp(r.standard_normal(n))[None, :]
    # gradients correlated with the inputs, so H is not itself a Kronecker product
    Xb = r.standard_normal((N, m)) * (1.0 + 0.5 * np.abs(Xa[:, :1]))
    return Xa, Xb


def test_kronecker_hessian_convention():
    # one sample: H = a a^T (x) b b^T = vecop(b a^T) vecop(b a^T)^T (column-major vec)
    a, b = np.array([1.0, 2.0]), np.array([3.0, -1.0, 0.5])
    G = np.outer(b, a)
    g = G.reshape(-1, order="F")
    assert np.allclose(dense.kronecker_hessian(a[None, :], b[None, :]), np.outer(g, g))


def test_frobenius_iteration_reaches_the_best_kronecker_product():
    # Van Loan-Pitsianis: min ||H - A (x) B||_F is the top singular pair of the
    # rearrangement R(H)[(i, j), (k, l)] = H[i m + k, j m + l] = A_ij B_kl.
    n, m = 3, 2
    Xa, Xb = _paired_samples(61, 40, n, m)
    H = dense.kronecker_hessian(Xa, Xb)
    R = H.reshape(n, m, n, m).transpose(0, 2, 1, 3).reshape(n * n, m * m)
    U, S, Vt = np.linalg.svd(R)
    best = S[0] * np.kron(U[:, 0].reshape(n, n), Vt[0].reshape(m, m))
    A, B = dense.kronecker_factors(Xa, Xb, "frobenius", 60)
    assert np.allclose(np.kron(A, B), best, rtol=0, atol=1e-9 * np.abs(best).max())
    # each half-step is a least-squares minimiser: perturbing A increases the residual
    res = np.linalg.norm(H - np.kron(A, B))
    for eps in (1e-3, -1e-3):
        assert np.linalg.norm(H - np.kron(A * (1 + eps), B)) > res


def test_flipflop_iterates_have_unit_mismatch_factor():
    # After every (undamped) B-update, tr(B^{-1} B) = m gives
    # E[(a^T A^{-1} a)(b^T B^{-1} b)] = m n, i.e. Phi(H, A (x) B) = 1 exactly.
    n, m = 3, 2
    Xa, Xb = _paired_samples(62, 50, n, m)
    H = dense.kronecker_hessian(Xa, Xb)
    for iters in (1, 2, 5):
        A, B = dense.kronecker_factors(Xa, Xb, "flipflop", iters)
        assert abs(dense.mismatch_factor(H, A, B) - 1.0) < 1e-12
    # the Frobenius approximation generally does not have Phi = 1
    A, B = dense.kronecker_factors(Xa, Xb, "frobenius", 5)
    assert abs(dense.mismatch_factor(H, A, B) - 1.0) > 1e-3


def test_flipflop_fixed_point_is_the_matrix_normal_mle():
    # The flip-flop fixed point maximises the matrix-normal likelihood of the
    # samples G_s = b_s a_s^T; compare with a generic optimiser of the negative
    # log-likelihood over Cholesky parametrisations of A and B (tiny sizes).
    from scipy.optimize import minimize
    n, m = 2, 2
    Xa, Xb = _paired_samples(63, 60, n, m)
    A, B = dense.kronecker_factors(Xa, Xb, "flipflop", 300)
    tri_n, tri_m = np.tril_indices(n), np.tril_indices(m)

    def unpack(p):
        La = np.zeros((n, n)); La[tri_n] = p[:len(tri_n[0])]
        Lb = np.zeros((m, m)); Lb[tri_m] = p[len(tri_n[0]):]
        La[np.diag_indices(n)] = np.exp(np.diag(La)); Lb[np.diag_indices(m)] = np.exp(np.diag(Lb))
        return La @ La.T, Lb @ Lb.T

    def nll(p):
        Ap, Bp = unpack(p)
        qa = np.einsum("si,ij,sj->s", Xa, np.linalg.inv(Ap), Xa)
        qb = np.einsum("si,ij,sj->s", Xb, np.linalg.inv(Bp), Xb)
        N = len(Xa)
        return 0.5 * (N * m * np.linalg.slogdet(Ap)[1] + N * n * np.linalg.slogdet(Bp)[1] + np.sum(qa * qb))

    res = minimize(nll, np.zeros(len(tri_n[0]) + len(tri_m[0])), method="BFGS", options={"gtol": 1e-10})
    Ao, Bo = unpack(res.x)
    K, Ko = np.kron(A, B), np.kron(Ao, Bo)
    assert np.allclose(K, Ko, rtol=1e-5, atol=1e-6 * np.abs(K).max())


def test_kronecker_factor_pins_catch_planted_mistakes():
    n, m = 3, 2
    Xa, Xb = _paired_samples(64, 50, n, m)
    H = dense.kronecker_hessian(Xa, Xb)
    N = len(Xa)
    # FlipFlop with the normalisers of the two factors swapped: Phi is off
    A, B = dense.kronecker_factors(Xa, Xb, "flipflop", 3)
    w = np.einsum("si,ij,sj->s", Xa, np.linalg.inv(A), Xa)
    B_bad = (Xb.T * w) @ Xb / (N * m)
    assert abs(dense.mismatch_factor(H, A, B_bad) - 1.0) > 1e-3
    # FlipFlop without the inverse (the Frobenius weighting) is not the MLE: Phi != 1
    A2, B2 = dense.kronecker_factors(Xa, Xb, "frobenius", 3)
    assert abs(dense.mismatch_factor(H, A2, B2) - 1.0) > 1e-3


# ------------------------------------------------------------ KronQ BiIP

def test_biip_scales_and_hadamard_match_printed_example():
    g = read_golden("kronq_biip_example.txt")
    sx = dense.biip_scales(np.diag(g["DIAG_H_X"][0]))
    sg = dense.biip_scales(np.diag(g["DIAG_H_G"][0]))
    assert np.array_equal(np.round(sx, 2), g["PRINTED_S_X"][0])
    assert np.array_equal(np.round(sg, 2), g["PRINTED_S_G"][0])
    Q = dense.biip_rotation(2, [1, 1])
    assert np.allclose(Q * np.sqrt(2), g["PRINTED_HADAMARD_TIMES_SQRT2"], atol=1e-15)


def test_biip_rotation_is_orthogonal():
    r = synth.rng(71)
    for d in (2, 48, 64, 96, 7):
        Q = dense.biip_rotation(d, np.where(r.random(d) < 0.5, -1.0, 1.0))
        assert np.allclose(Q.T @ Q, np.eye(d), atol=1e-13)
    assert dense.hadamard_block(14336) == 2048 and dense.hadamard_block(4096) == 4096
    assert dense.hadamard_block(65536) == dense.BIIP_MAX_BLOCK and dense.hadamard_block(7) == 1


def _biip_problem(seed, m, n):
    c = synth.spectral(m, n, config=seed)
    r = synth.rng(seed + 77)
    sn = np.where(r.random(n) < 0.5, -1.0, 1.0)
    sm = np.where(r.random(m) < 0.5, -1.0, 1.0)
    # distinct diagonal magnitudes, so the rescale matters
    A = c["A"] * np.outer(np.linspace(1, 3, n), np.linspace(1, 3, n))
    B = c["B"] * np.outer(np.linspace(2, 0.5, m), np.linspace(2, 0.5, m))
    return c["W"], A, B, sn, sm


def test_biip_loss_is_invariant():
    # KronQ page Theorem 1 (orthogonal rotations) together with the paired
    # diagonal rescale: for any V'' in the processed coordinates,
    # tr(B E A E^T) with E = inverse(V'') - W equals tr(B'' E'' A'' E''^T).
    W, A, B, sn, sm = _biip_problem(81, 24, 40)
    W2, A2, B2, sa, sb = dense.biip_forward(W, A, B, sn, sm)
    V2 = W2 + 0.1 * synth.gaussian(82, W2.shape)
    V = dense.biip_inverse(V2, sn, sm, sa, sb)
    l2 = dense.proxy_loss(W2, V2, A2, B2)
    assert abs(dense.proxy_loss(W, V, A, B) - l2) <= 1e-12 * l2
    assert np.allclose(dense.biip_inverse(W2, sn, sm, sa, sb), W, atol=1e-12)
    # planted mistake: factors scaled by S instead of S^{-1} break the invariance
    A_bad = dense.biip_rotation(40, sn) @ (A * np.outer(sa, sa)) @ dense.biip_rotation(40, sn).T
    assert abs(dense.proxy_loss(W2, V2, A_bad, B2) - l2) > 1e-3 * l2


def test_biip_spreads_an_outlier():
    W = 0.01 * synth.gaussian(83, (32, 64))
    W[5, 7] = 10.0
    A, B = np.eye(64), np.eye(32)
    W2 = dense.biip_forward(W, A, B, np.ones(64), np.ones(32))[0]
    peak = lambda M: np.abs(M).max() / np.sqrt(np.mean(M ** 2))
    assert peak(W2) < 0.1 * peak(W)
