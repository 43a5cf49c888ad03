"""GPU parity of the KronQ BiIP transforms (KronQ page, section
"Kronecker-Factored Quantization") through the C ABI, against the oracle's
dense-matrix form (explicit Walsh-Hadamard matrices).

Bars: transformed W, A, B and the scales to 1e-12 (fp64) / 2e-6 (fp32)
relative max-norm; the round trip inverse(forward(W)) = W; and, the point of
Theorem 1, the whole path run on the processed problem (prepare, two-sided
GPTQ, back-transform) gives a V whose loss in the original coordinates equals
the processed problem's loss (kron_loss on both sides, fp64 1e-10).
"""
import numpy as np
import pytest

import synth
from oracle import dense

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import two_sided_gptq_damped_amd as kq  # noqa: E402
from two_sided_gptq_damped_amd import pipeline  # noqa: E402

DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def up(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a).astype(dtype))).to(DEV)


def problem(seed, m, n):
    c = synth.spectral(m, n, config=seed)
    r = synth.rng(seed + 77)
    sn = np.where(r.random(n) < 0.5, -1, 1).astype(np.int8)
    sm = np.where(r.random(m) < 0.5, -1, 1).astype(np.int8)
    A = c["A"] * np.outer(np.linspace(1, 3, n), np.linspace(1, 3, n))
    B = c["B"] * np.outer(np.linspace(2, 0.5, m), np.linspace(2, 0.5, m))
    return c["W"], A, B, sn, sm


def gpu_forward(W, A, B, sn, sm, dtype):
    m, n = W.shape
    t = lambda a: up(a, dtype)
    Wt, At, Bt = t(W), t(A), t(B)
    Wo, Ao, Bo = torch.empty_like(Wt), torch.empty_like(At), torch.empty_like(Bt)
    sa = torch.empty(n, dtype=Wt.dtype, device=DEV)
    sb = torch.empty(m, dtype=Wt.dtype, device=DEV)
    ws = kq.biip_workspace(Wt.dtype, m, n)
    sn_t, sm_t = torch.from_numpy(sn).to(DEV), torch.from_numpy(sm).to(DEV)
    kq.kron_biip_forward(Wt, At, Bt, sn_t, sm_t, Wo, Ao, Bo, sa, sb, ws)
    return Wo, Ao, Bo, sa, sb, sn_t, sm_t, ws


def rel(X, Y):
    return float(np.max(np.abs(np.asarray(X, dtype=np.float64) - Y)) / np.max(np.abs(Y)))


@pytest.mark.parametrize("m,n", [(64, 48), (96, 80), (130, 70), (256, 256), (48, 7), (14, 4096), (1024, 4096)])
def test_biip_forward_matches_oracle(m, n):
    W, A, B, sn, sm = problem(30 + m % 7, m, n)
    for dtype, tol in ((np.float64, 1e-12), (np.float32, 2e-6)):
        Wd, Ad, Bd = (x.astype(dtype).astype(np.float64) for x in (W, A, B))
        W2, A2, B2, sa, sb = dense.biip_forward(Wd, Ad, Bd, sn, sm)
        Wo, Ao, Bo, sag, sbg, sn_t, sm_t, ws = gpu_forward(W, A, B, sn, sm, dtype)
        h = lambda t: t.cpu().numpy()
        errs = [rel(h(Wo), W2), rel(h(Ao), A2), rel(h(Bo), B2), rel(h(sag), sa), rel(h(sbg), sb)]
        say("biip", (m, n), np.dtype(dtype).name, " ".join(f"{e:.1e}" for e in errs))
        assert max(errs) <= tol
        back = torch.empty_like(Wo)
        kq.kron_biip_inverse(Wo, sn_t, sm_t, sag, sbg, back, ws)
        assert rel(h(back), Wd) <= tol


def test_biip_quantization_loss_is_invariant():
    # Theorem 1 on the whole path: process, prepare the processed factors, run
    # two-sided GPTQ on W'', map V'' back; the original-coordinate loss of V
    # equals the processed problem's loss.
    m, n = 256, 192
    W, A, B, sn, sm = problem(41, m, n)
    Wo, Ao, Bo, sa, sb, sn_t, sm_t, ws = gpu_forward(W, A, B, sn, sm, np.float64)
    UA, _, _ = pipeline.prepare(Ao, 0.0)
    UB, _, _ = pipeline.prepare(Bo, 0.0)
    codes, V2, _ = pipeline.quantize(Wo, UA, UB, 3, True)
    V = torch.empty_like(V2)
    kq.kron_biip_inverse(V2, sn_t, sm_t, sa, sb, V, ws)
    l_proc = pipeline.loss(Wo, V2, Ao, Bo, 0.0).item()
    l_orig = pipeline.loss(up(W, np.float64), V, up(A, np.float64), up(B, np.float64), 0.0).item()
    say("biip loss", f"processed {l_proc:.10e} original {l_orig:.10e}")
    assert abs(l_orig - l_proc) <= 1e-10 * l_proc
