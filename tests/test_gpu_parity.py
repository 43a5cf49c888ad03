"""GPU parity: every entry point through the C ABI against the CPU oracle.

Inputs are the seeded synthetic workloads of synth/.  For kron_quantize the
factors U_A, U_B come from the oracle's fp64 preparation and are rounded to the
run dtype; both sides then solve the same problem:
  fp64: codes equal, except at entries whose oracle pre-rounding value lies
        within 1e-9 grid units of a rounding midpoint (handled by re-running the
        oracle with the GPU's code imposed there); V equal where codes are equal.
  fp32: code mismatch fraction <= 1e-3 and proxy-loss relative error <= 1e-3
        against the fp64 oracle on the fp32-rounded inputs.
The other entry points are compared with the oracle's definitions within
tolerances derived from their arithmetic (stated per test).
"""
import numpy as np
import pytest

import synth
from oracle import compare, dense, o3

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import two_sided_gptq_damped_amd as kq  # noqa: E402
from two_sided_gptq_damped_amd import pipeline  # noqa: E402

DEV = "cuda"
TORCH_DT = {np.float64: torch.float64, np.float32: torch.float32}


def say(*a):
    print("[case]", *a, flush=True)


def up(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a).astype(dtype))).to(DEV)


def oracle_factors(A, B, delta=0.01):
    Ad, UA = dense.prepare(A, delta)
    Bd, UB = (None, None) if B is None else dense.prepare(B, delta)
    return Ad, UA, Bd, UB


def gpu_quantize(W, UA, UB, s, bits, per_row, dtype):
    Wt, UAt = up(W, dtype), up(UA, dtype)
    UBt = None if UB is None else up(UB, dtype)
    st = up(s, dtype)
    codes, V, _ = pipeline.quantize(Wt, UAt, UBt, bits, per_row, scales=st)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), V.cpu().numpy()


def check_fp64(W, UA, UB, s, bits, per_row, label):
    say(label, "fp64", W.shape)
    Zg, Vg = gpu_quantize(W, UA, UB, s, bits, per_row, np.float64)
    run = lambda f: o3.solve(W, UA, UB, s, bits, force=f)[0::2]
    ok, nforced, info = compare.codes_equal_up_to_ties(Zg, run)
    assert ok, f"{label}: {info}"
    Zo, Vo, _, _ = o3.solve(W, UA, UB, s, bits)
    same = Zo == Zg
    assert np.array_equal(Vg[same], Vo[same])
    return Zg, Vg


def check_fp32(W, UA, UB, s, bits, per_row, Ad, Bd, label, max_mis=1e-3, max_loss=1e-3):
    say(label, "fp32", W.shape)
    W32, UA32 = W.astype(np.float32), UA.astype(np.float32)
    UB32 = None if UB is None else UB.astype(np.float32)
    s32 = np.asarray(s).astype(np.float32)
    Zg, Vg = gpu_quantize(W32, UA32, UB32, s32, bits, per_row, np.float32)
    Zo, Vo, _, _ = o3.solve(W32.astype(np.float64), UA32.astype(np.float64),
                            None if UB is None else UB32.astype(np.float64), s32.astype(np.float64), bits)
    mis = compare.mismatch_fraction(Zg, Zo)
    Bl = np.eye(W.shape[0]) if Bd is None else Bd
    lg = dense.proxy_loss(W32.astype(np.float64), Vg.astype(np.float64), Ad, Bl)
    lo = dense.proxy_loss(W32.astype(np.float64), Vo, Ad, Bl)
    rel = compare.rel_diff(lg, lo)
    say(label, f"mismatch={mis:.3e} loss_rel={rel:.3e}")
    assert mis <= max_mis and rel <= max_loss
    return Zg, Vg


# ---------------------------------------------------------------- the solver

def test_tiny_fp64_matches_literal_kronecker_gptq():
    c = synth.tiny()
    A = dense.factor_accumulate(c["act"], alpha=1 / 256)
    B = dense.factor_accumulate(c["grad"], alpha=1 / 256)
    Ad, UA, Bd, UB = oracle_factors(A, B)
    s = dense.scales(c["W"], 4, False)
    Zg, Vg = check_fp64(c["W"], UA, UB, s, 4, False, "tiny 32x32")
    Z1, V1, Y1 = dense.vectorized_kron_gptq(c["W"], Ad, Bd, s, 4)
    assert np.array_equal(Zg, Z1)
    lg = dense.proxy_loss(c["W"], Vg, Ad, Bd)
    assert abs(lg - dense.proxy_loss(c["W"], V1, Ad, Bd)) <= 1e-12 * lg


@pytest.fixture(scope="module")
def spectral():
    c = synth.spectral()
    Ad, UA, Bd, UB = oracle_factors(c["A"], c["B"])
    s = dense.scales(c["W"], 3, True)
    return c, Ad, UA, Bd, UB, s


def test_spectral_256_fp64(spectral):
    c, Ad, UA, Bd, UB, s = spectral
    check_fp64(c["W"], UA, UB, s, 3, True, "spectral 256")


def test_spectral_256_fp32(spectral):
    c, Ad, UA, Bd, UB, s = spectral
    check_fp32(c["W"], UA, UB, s, 3, True, Ad, Bd, "spectral 256")


def test_spectral_256_b_identity_is_one_sided_gptq(spectral):
    c, Ad, UA, Bd, UB, s = spectral
    say("spectral 256 B=I")
    Zg, Vg = gpu_quantize(c["W"], UA, None, s, 3, True, np.float64)
    Zr, Vr = dense.one_sided_gptq(c["W"], UA, s, 3)
    Yr = o3.solve(c["W"], UA, None, s, 3)[2]
    assert np.all((Zg == Zr) | (compare.tie_distance(Yr) < 1e-9))
    check_fp32(c["W"], UA, None, s, 3, True, Ad, None, "spectral 256 B=I")


@pytest.mark.parametrize("m,n", [(100, 70), (64, 130), (1, 50), (50, 1), (65, 65), (127, 129), (3, 200),
                                 (192, 64)])
def test_ragged_shapes_fp64(m, n):
    c = synth.spectral(m, n, config=2)
    _, UA, _, UB = oracle_factors(c["A"], c["B"])
    s = dense.scales(c["W"], 4, True)
    check_fp64(c["W"], UA, UB, s, 4, True, f"ragged {m}x{n}")


def test_tall_one_sided_at_the_largest_m():
    # m = 65536, the largest the ABI takes: the solver's set-up kernels walk the
    # rows past the 65535 that one grid dimension holds, and the leaves run 2049
    # tile-diagonals of at most two tiles.  B = I, so no 65536^2 output factor.
    m, n = 65536, 64
    W = synth.gaussian(401, (m, n))
    A = dense.factor_accumulate(synth.channel_scaled_rows(402, 403, 256, n), alpha=1 / 256)
    _, UA, _, _ = oracle_factors(A, None)
    s = dense.scales(W, 3, True)
    check_fp64(W, UA, None, s, 3, True, "tall one-sided")


@pytest.mark.parametrize("bits,per_row", [(2, True), (3, False), (5, True), (8, False)])
def test_bits_and_scale_modes(bits, per_row):
    c = synth.spectral(96, 80, config=2)
    Ad, UA, Bd, UB = oracle_factors(c["A"], c["B"])
    s = dense.scales(c["W"], bits, per_row)
    check_fp64(c["W"], UA, UB, s, bits, per_row, f"bits={bits} per_row={per_row}")
    check_fp32(c["W"], UA, UB, s, bits, per_row, Ad, Bd, f"bits={bits} per_row={per_row}")


def test_zero_row_scale_gives_zero_codes():
    c = synth.spectral(64, 64, config=2)
    _, UA, _, UB = oracle_factors(c["A"], c["B"])
    W = c["W"].copy()
    W[5, :] = 0.0
    s = dense.scales(W, 3, True)
    Zg, Vg = check_fp64(W, UA, UB, s, 3, True, "zero row")
    assert np.all(Zg[5] == 0) and np.all(Vg[5] == 0)


@pytest.mark.parametrize("per_row", [True, False])
def test_identity_factors_round_to_nearest_with_exact_ties(per_row):
    # A = B = I: no feedback reaches any entry, so two-sided GPTQ is round to
    # nearest (FastKron page section 2.2 with identity curvature).  Every entry is
    # an exact half-integer multiple of a power-of-two scale, so the GPU's
    # rounding must be round-half-to-even at every entry, with no tie tolerance.
    m, n, bits = 96, 80, 4
    r = synth.rng(4242)
    e = r.integers(-6, 3, size=m)
    s = np.ldexp(1.0, e) if per_row else np.full(m, 0.125)
    k = r.integers(-8, 8, size=(m, n)).astype(np.float64) + 0.5  # half-integers, some beyond the grid
    k[:, 0] = 7.0  # the row maximum: max |W_i| / 7 is exactly s_i
    k = np.clip(k, -7.0, 7.0)
    W = k * s[:, None]
    sc = dense.scales(W, bits, per_row)
    assert np.array_equal(dense.row_scales(sc, m), s)
    want = np.clip(np.rint(k), -8, 7)
    assert np.sum(want != np.floor(k)) > 0 and np.sum(np.abs(k - np.floor(k) - 0.5) == 0) > m * n // 2
    for dtype in (np.float64, np.float32):
        for UB in (np.eye(m), None):
            Zg, Vg = gpu_quantize(W, np.eye(n), UB, sc, bits, per_row, dtype)
            say("rtn ties", np.dtype(dtype).name, "B=I" if UB is None else "two-sided", per_row)
            assert np.array_equal(Zg.astype(np.float64), want)
            assert np.array_equal(Vg.astype(np.float64), want * s[:, None])


def test_exact_tie_at_the_first_entry():
    # Entry (0, 0) receives no feedback, so x_00 = W_00 exactly; with W_00 = 2.5 s_0
    # and s_0 a power of two both sides see an exact tie, which rounds to the even
    # code 2.  Asserted without a tie tolerance, two-sided and B = I, fp64 and fp32.
    c = synth.spectral(64, 64, config=2)
    _, UA, _, UB = oracle_factors(c["A"], c["B"])
    W = c["W"].copy()
    W[0, :] = np.clip(W[0, :], -1.5, 1.5)
    W[0, 5] = 1.75  # max |W_0| / 7 = 0.25
    W[0, 0] = 2.5 * 0.25
    s = dense.scales(W, 4, True)
    assert s[0] == 0.25
    for UBx in (UB, None):
        Zo, _, Yo, _ = o3.solve(W, UA, UBx, s, 4)
        assert Zo[0, 0] == 2 and Yo[0, 0] == 2.5
        for dtype in (np.float64, np.float32):
            Wd = W.astype(dtype).astype(np.float64)
            Zg, Vg = gpu_quantize(Wd, UA, UBx, s, 4, True, dtype)
            say("tie at origin", np.dtype(dtype).name, "B=I" if UBx is None else "two-sided")
            assert Zg[0, 0] == 2 and Vg[0, 0] == 0.5
            if dtype == np.float64:
                assert np.array_equal(Zg, Zo)


def test_deterministic_replay(spectral):
    c, Ad, UA, Bd, UB, s = spectral
    say("replay")
    a = gpu_quantize(c["W"], UA, UB, s, 3, True, np.float32)
    b = gpu_quantize(c["W"], UA, UB, s, 3, True, np.float32)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------- other entry points

def _check_prepare(A, label, tol64=1e-9, tol32=1e-5):
    """kron_prepare against the oracle's damped factor (route (i): inverse, then
    Cholesky), fp64 and fp32, plus U^T U A_d = I for the fp64 result."""
    for dtype, tol in ((np.float64, tol64), (np.float32, tol32)):
        Ar = A.astype(dtype)
        U, tr, lam = pipeline.prepare(up(Ar, dtype), 0.01)
        U = U.cpu().numpy().astype(np.float64)
        Ad, Uo = dense.prepare(Ar.astype(np.float64), 0.01)
        err = np.max(np.abs(U - Uo)) / np.max(np.abs(Uo))
        say(label, np.dtype(dtype).name, f"max |U - U_oracle| / max |U_oracle| = {err:.2e}")
        assert err <= tol, label
        assert np.all(np.tril(U, -1) == 0)
        assert abs(tr.item() - np.trace(Ar.astype(np.float64))) <= 1e-12 * abs(np.trace(A))
        assert abs(lam.item() - 0.01 * np.trace(Ar.astype(np.float64)) / len(A)) <= 1e-12 * abs(lam.item())
        if dtype == np.float64:
            res = np.max(np.abs(U.T @ U @ Ad - np.eye(len(A))))
            say(label, f"max |U^T U A_d - I| = {res:.2e}")
            assert res <= 1e-6, label


# d = 320, 1000: several four-block Cholesky panels (the cross-panel trailing
# update) and the deeper levels of the recursive triangular inverse, with a
# ragged last tile at 1000.
@pytest.mark.parametrize("d", [1, 17, 64, 100, 256, 320, 1000])
def test_prepare_matches_oracle(d):
    say("prepare", d)
    c = synth.spectral(d, d, config=2)
    _check_prepare(c["A"], f"prepare spectral {d}")


@pytest.mark.timeout(300)
def test_prepare_matches_oracle_llm_4096():
    # The workload's own factor: A = X^T X / 4096 from 4096 channel-scaled rows
    # (lognormal channel scales), the 4096 x 4096 input factor of the 4096^2 layer.
    say("prepare llm 4096")
    X = synth.channel_scaled_rows(3003, 3004, 4096, 4096)
    A = dense.factor_accumulate(X, alpha=1.0 / 4096)
    _check_prepare(A, "prepare llm 4096")


def test_prepare_detects_indefinite():
    say("prepare indefinite")
    A = -np.eye(32)
    A[3, 3] = 2.0
    At = up(A, np.float64)
    with pytest.raises(kq.KronError) as e:
        pipeline.prepare(At, 0.0)
    assert e.value.status == 2
    info = torch.zeros(1, dtype=torch.int32, device=DEV)
    U = torch.empty_like(At)
    ws = kq.workspace(kq.KQ_OP_PREPARE, torch.float64, 32, 0)
    kq.kron_prepare(At, 0.0, U, ws, info=info)
    torch.cuda.synchronize()
    assert info.item() == 1  # the last index of A is the first pivot of the reversed factorisation


@pytest.mark.parametrize("rows,dim", [(256, 32), (300, 100), (4096, 256), (7, 65)])
def test_factor_accumulate(rows, dim):
    say("factor", rows, dim)
    X = synth.channel_scaled_rows(77, 78, rows, dim)
    S0 = synth.gaussian(79, (dim, dim))
    for dtype, tol in ((np.float64, 1e-12), (np.float32, 1e-5)):
        Xt, St = up(X, dtype), up(S0, dtype)
        kq.kron_factor_accumulate(Xt, St, 1.0 / rows, 0.5)
        want = dense.factor_accumulate(X.astype(dtype).astype(np.float64), S0.astype(dtype), 1.0 / rows, 0.5)
        got = St.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got - want)) <= tol * np.max(np.abs(want))


# (n <= m: the m x m form E A_d E^T; n > m: the n x n form E^T B_d E; several
# tiles of the symmetric product with ragged edges; B = I)
@pytest.mark.parametrize("m,n,bidentity", [(32, 32, False), (100, 70, False), (200, 130, False), (130, 300, False),
                                           (256, 256, False), (64, 130, True), (300, 90, True)])
def test_loss_matches_oracle(m, n, bidentity):
    say("loss", m, n)
    c = synth.spectral(m, n, config=2)
    V = c["W"] + 0.1 * synth.gaussian(91, (m, n))
    for dtype in (np.float64, np.float32):
        W32, V32 = c["W"].astype(dtype), V.astype(dtype)
        B = None if bidentity else c["B"].astype(dtype)
        got = pipeline.loss(up(W32, dtype), up(V32, dtype), up(c["A"], dtype),
                            None if B is None else up(B, dtype), 0.01).item()
        Ad = dense.damp(c["A"].astype(dtype).astype(np.float64), 0.01)
        Bd = np.eye(m) if B is None else dense.damp(B.astype(np.float64), 0.01)
        want = dense.proxy_loss(W32.astype(np.float64), V32.astype(np.float64), Ad, Bd)
        assert abs(got - want) <= 1e-12 * abs(want)


# kron_quantize's own proxy loss (from its rounding errors) against kron_loss on
# its output, the trace form from W and V alone.  The two agree up to the rounding
# of the solver's feedback sums: fp64 1e-10 relative, fp32 1e-4 (the identity
# V - W = L~_B Delta L~_A^T holds for exact sums; fp32 sums carry ~1e-7 relative
# error per entry and the fp32-rounded U only approximates the factor of A_d).
@pytest.mark.parametrize("m,n,two_sided", [(32, 32, True), (100, 70, True), (130, 300, False), (256, 256, True),
                                           (300, 90, True)])
def test_quantize_loss_matches_trace_form(m, n, two_sided):
    say("quantize loss", m, n, two_sided)
    c = synth.spectral(m, n, config=2)
    _, UA, _, UB = oracle_factors(c["A"], c["B"] if two_sided else None)
    s = dense.scales(c["W"], 3, True)
    for dtype, tol in ((np.float64, 1e-10), (np.float32, 1e-4)):
        Wt, st = up(c["W"], dtype), up(s, dtype)
        lo = torch.zeros(1, dtype=torch.float64, device=DEV)
        _, V, _ = pipeline.quantize(Wt, up(UA, dtype), up(UB, dtype) if two_sided else None, 3, True, scales=st,
                                    loss_out=lo)
        trace = pipeline.loss(Wt, V, up(c["A"], dtype), up(c["B"], dtype) if two_sided else None, 0.01).item()
        got = lo.item()
        say("  ", dtype.__name__, got, trace, abs(got - trace) / trace)
        assert trace > 0 and abs(got - trace) <= tol * trace


@pytest.mark.parametrize("per_row", [True, False])
def test_row_scales_bit_exact(per_row):
    say("scales", per_row)
    W = synth.heavy_weight(5, 6, 130, 257)
    for dtype in (np.float64, np.float32):
        Wt = up(W, dtype)
        s = torch.empty(130 if per_row else 1, dtype=TORCH_DT[dtype], device=DEV)
        kq.kron_row_scales(Wt, 3, per_row, s)
        want = dense.scales(W.astype(dtype).astype(np.float64), 3, per_row).astype(dtype)
        assert np.array_equal(s.cpu().numpy(), want)


@pytest.mark.parametrize("two_sided", [True, False])
def test_pipelined_layers_equal_one_at_a_time(two_sided):
    # quantize_layers overlaps layer k + 1's factor chains with layer k's solve
    # and solves consecutive layers on two streams at once; every result must
    # equal quantize_layer on that layer alone, bit for bit (the path is
    # deterministic), across shapes that change from layer to layer (the last
    # two large enough for both solves' band products to fill the GPU together).
    say("pipelined layers", two_sided)
    shapes = [(96, 64), (64, 130), (100, 100), (33, 70), (520, 384), (384, 640)]
    for dtype in (np.float64, np.float32):
        layers = []
        for i, (m, n) in enumerate(shapes):
            layers.append((up(synth.gaussian(300 + i, (m, n)), dtype),
                           up(synth.channel_scaled_rows(310 + i, 320 + i, 256, n), dtype),
                           up(synth.channel_scaled_rows(330 + i, 340 + i, 256, m), dtype)))
        piped = pipeline.quantize_layers(layers, bits=3, two_sided=two_sided)
        for (W, act, grad), got in zip(layers, piped):
            want = pipeline.quantize_layer(W, act, grad, bits=3, two_sided=two_sided)
            assert torch.equal(got["codes"], want["codes"])
            assert torch.equal(got["V"], want["V"])
            assert got["loss"].item() == want["loss"].item()
            assert torch.equal(got["U_A"], want["U_A"])


def test_pipeline_tiny_all_on_gpu_fp64():
    # Every step on the GPU (factor, prepare, scales, quantize, loss) against the
    # oracle's own pipeline on the same samples; factors differ only by rounding.
    say("pipeline tiny fp64")
    c = synth.tiny()
    out = pipeline.quantize_layer(up(c["W"], np.float64), up(c["act"], np.float64), up(c["grad"], np.float64),
                                  bits=4, per_row=False, check_loss=True)
    A = dense.factor_accumulate(c["act"], alpha=1 / 256)
    B = dense.factor_accumulate(c["grad"], alpha=1 / 256)
    Ad, UA, Bd, UB = oracle_factors(A, B)
    s = dense.scales(c["W"], 4, False)
    Zo, Vo, Yo, _ = o3.solve(c["W"], UA, UB, s, 4)
    Zg = out["codes"].cpu().numpy()
    assert np.all((Zg == Zo) | (compare.tie_distance(Yo) < 1e-9))
    lo = dense.proxy_loss(c["W"], Vo, Ad, Bd)
    assert abs(out["loss"].item() - lo) <= 1e-10 * lo  # from the solver's errors
    assert abs(out["loss_check"].item() - lo) <= 1e-10 * lo  # kron_loss on W and V
    assert abs(out["trace_A"].item() * out["trace_B"].item() - dense.sensitivity(A, B)) <= 1e-12 * dense.sensitivity(A, B)
