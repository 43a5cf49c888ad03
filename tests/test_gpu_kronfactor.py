"""GPU parity of kron_factor_kronecker (FlipFlop and Frobenius Kronecker
approximations of H = E[a a^T (x) b b^T], WaterKron page section 5 and Table 1)
through the C ABI, against the oracle's iteration on the same paired samples.

Tolerances (relative max-norm of each factor): fp64 1e-10 (the same operations
in another summation order, through one damped inverse per half-step); fp32
2e-4 (fp32 products and SYRK, the quadratic forms through fp32-rounded factors
of condition up to ~1e4).
"""
import time

import numpy as np
import pytest

import synth
from oracle import dense

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import two_sided_gptq_damped_amd as kq  # noqa: E402

DEV = "cuda"
METHODS = {"flipflop": kq.KQ_KRON_FLIPFLOP, "frobenius": kq.KQ_KRON_FROBENIUS}


def say(*a):
    print("[case]", *a, flush=True)


def up(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a).astype(dtype))).to(DEV)


def samples(seed, N, n, m):
    """Paired activation / gradient rows: channel-scaled activations and gradients
    whose scale depends on the sample's activation (so H is not a Kronecker product)."""
    Xa = synth.channel_scaled_rows(seed, seed + 1, N, n)
    g = synth.channel_scaled_rows(seed + 2, seed + 3, N, m)
    return Xa, g * (1.0 + 0.5 * np.abs(Xa[:, :1]) / np.abs(Xa[:, :1]).mean())


def gpu_factors(Xa, Xb, method, iters, damp, dtype):
    N, n = Xa.shape
    m = Xb.shape[1]
    tdt = torch.float64 if dtype == np.float64 else torch.float32
    A = torch.empty(n, n, dtype=tdt, device=DEV)
    B = torch.empty(m, m, dtype=tdt, device=DEV)
    ws = kq.kronecker_workspace(tdt, N, n, m)
    kq.kron_factor_kronecker(up(Xa, dtype), up(Xb, dtype), METHODS[method], iters, damp, A, B, ws)
    torch.cuda.synchronize()
    return A.cpu().numpy().astype(np.float64), B.cpu().numpy().astype(np.float64)


def rel(X, Y):
    return float(np.max(np.abs(X - Y)) / np.max(np.abs(Y)))


@pytest.mark.parametrize("method", ["flipflop", "frobenius"])
@pytest.mark.parametrize("N,n,m,iters", [(512, 96, 80, 1), (1000, 130, 70, 2), (4096, 256, 320, 3), (300, 65, 1, 2)])
def test_kronecker_factors_match_oracle(method, N, n, m, iters):
    Xa, Xb = samples(700 + n, N, n, m)
    for dtype, tol in ((np.float64, 1e-10), (np.float32, 2e-4)):
        Xa_d, Xb_d = Xa.astype(dtype).astype(np.float64), Xb.astype(dtype).astype(np.float64)
        A, B = gpu_factors(Xa, Xb, method, iters, 0.01, dtype)
        Ao, Bo = dense.kronecker_factors(Xa_d, Xb_d, method, iters, 0.01)
        ea, eb = rel(A, Ao), rel(B, Bo)
        say(method, np.dtype(dtype).name, (N, n, m, iters), f"rel err A {ea:.2e} B {eb:.2e}")
        assert ea <= tol and eb <= tol
        assert np.array_equal(A, A.T) and np.array_equal(B, B.T)


def test_flipflop_gpu_factors_have_unit_mismatch_factor():
    # undamped FlipFlop: Phi(H, A (x) B) = tr(H (A (x) B)^{-1}) / (m n) = 1 after
    # every B-update (WaterKron page section 4), checked against the explicit H
    Xa, Xb = samples(801, 400, 6, 5)
    H = dense.kronecker_hessian(Xa, Xb)
    for iters in (1, 3):
        A, B = gpu_factors(Xa, Xb, "flipflop", iters, 0.0, np.float64)
        phi = dense.mismatch_factor(H, A, B)
        say("flipflop phi", iters, phi)
        assert abs(phi - 1.0) < 1e-10


@pytest.mark.timeout(300)
def test_flipflop_llm_4096_fp32():
    # the 4096 x 4096 layer's calibration shape: 4096 paired rows, two FlipFlop
    # iterations (the WaterKron page finds the second iteration helps), fp32
    Xa, Xb = samples(901, 4096, 4096, 4096)
    t = time.perf_counter()
    A, B = gpu_factors(Xa, Xb, "flipflop", 2, 0.01, np.float32)
    say("flipflop 4096 fp32 wall incl. transfers", f"{time.perf_counter() - t:.3f} s")
    Xa32, Xb32 = (x.astype(np.float32).astype(np.float64) for x in (Xa, Xb))
    say("flipflop 4096: oracle (fp64, CPU)")
    Ao, Bo = dense.kronecker_factors(Xa32, Xb32, "flipflop", 2, 0.01)
    ea, eb = rel(A, Ao), rel(B, Bo)
    say("flipflop 4096 fp32", f"rel err A {ea:.2e} B {eb:.2e}")
    assert ea <= 2e-4 and eb <= 2e-4
