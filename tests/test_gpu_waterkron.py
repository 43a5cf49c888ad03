"""GPU parity of the WaterKron mode (WaterKron page, sections 2.1, 2.4 and 3)
through the C ABI: kron_waterkron_scales against the oracle's definition, and
kron_quantize_waterkron (per-entry steps beta_i alpha_j, unbounded int32 codes)
against the oracle's left-looking loop with the same steps.

Bars as for kron_quantize: fp64 codes equal except at oracle pre-rounding
values within 1e-9 grid units of a midpoint (V equal where codes are equal);
fp32 codes checked along the GPU's own trajectory (1e-4 grid units), every
mismatch root a near tie, the near-tie branches at most four times those of
the oracle's own fp32 loop (at least two counted), mismatch <= 1e-3 when the
GPU took no branch, and loss within 1e-3 of the fp64 oracle.  At 4096 x 4096 the run also reports the empirical entropy of the
codes and the high-rate distortion ratio loss / (m n step^2 / 12).
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


def say(*a):
    print("[case]", *a, flush=True)


def up(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a).astype(dtype))).to(DEV)


def gpu_scales(UA, UB, step, m):
    n = UA.shape[0]
    alpha = torch.empty(n, dtype=UA.dtype, device=DEV)
    beta = torch.empty(m, dtype=UA.dtype, device=DEV)
    kq.kron_waterkron_scales(UA, UB, step, alpha, beta)
    return alpha, beta


def gpu_waterkron(W, UA, UB, alpha, beta, loss=None):
    m, n = W.shape
    codes = torch.empty(m, n, dtype=torch.int32, device=DEV)
    V = torch.empty_like(W)
    ws = kq.workspace(kq.KQ_OP_QUANTIZE, W.dtype, m, n)
    kq.kron_quantize_waterkron(W, UA, UB, alpha, beta, codes, V, ws, loss=loss)
    return codes, V


def transformed_rms(W, UA, UB):
    """Spread of W / (U_B,ii U_A,jj): a natural unit for the WaterKron step."""
    dB = np.ones(W.shape[0]) if UB is None else np.diag(UB)
    return float(np.sqrt(np.mean((W / np.outer(dB, np.diag(UA))) ** 2)))


@pytest.mark.parametrize("two_sided", [True, False])
def test_waterkron_scales_match_definition(two_sided):
    c = synth.spectral(96, 80, config=2)
    _, UA = dense.prepare(c["A"], 0.01)
    _, UB = dense.prepare(c["B"], 0.01)
    for dtype in (np.float64, np.float32):
        Ud_A, Ud_B = UA.astype(dtype), UB.astype(dtype)
        alpha, beta = gpu_scales(up(Ud_A, dtype), up(Ud_B, dtype) if two_sided else None, 0.37, 96)
        wa, wb = dense.waterkron_scales(Ud_A.astype(np.float64), Ud_B.astype(np.float64) if two_sided else None,
                                        0.37, m=96)
        assert np.array_equal(alpha.cpu().numpy(), wa.astype(dtype))
        assert np.array_equal(beta.cpu().numpy(), wb.astype(dtype))


def check_fp64(W, UA, UB, step, label):
    m, n = W.shape
    alpha, beta = dense.waterkron_scales(UA, UB, step, m=m)
    Zg, Vg = gpu_waterkron(up(W, np.float64), up(UA, np.float64), None if UB is None else up(UB, np.float64),
                           up(alpha, np.float64), up(beta, np.float64))
    Zg, Vg = Zg.cpu().numpy(), Vg.cpu().numpy()
    run = lambda f: o3.solve(W, UA, UB, beta, None, force=f, alpha=alpha)[0::2]
    ok, nforced, info = compare.codes_equal_up_to_ties(Zg, run)
    Zo, Vo, _, _ = o3.solve(W, UA, UB, beta, None, alpha=alpha)
    say(label, f"fp64 {m}x{n}: equal={ok} forced={nforced} max|code|={int(np.abs(Zo).max())} "
               f"entropy={dense.empirical_entropy(Zo):.3f} bits")
    assert ok, f"{label}: {info}"
    same = Zo == Zg
    assert np.array_equal(Vg[same], Vo[same])
    return Zg


@pytest.mark.parametrize("m,n,two_sided", [(256, 256, True), (100, 70, True), (65, 65, True), (127, 129, True),
                                           (1, 50, True), (50, 1, True), (96, 80, False), (384, 640, False),
                                           (520, 384, True), (1024, 1024, True), (256, 1536, False)])
def test_waterkron_fp64_matches_oracle(m, n, two_sided):
    c = synth.spectral(m, n, config=2)
    _, UA = dense.prepare(c["A"], 0.01)
    UB = dense.prepare(c["B"], 0.01)[1] if two_sided else None
    step = 0.5 * transformed_rms(c["W"], UA, UB)
    check_fp64(c["W"], UA, UB, step, f"waterkron {m}x{n} {'two-sided' if two_sided else 'WaterSIC'}")


def test_waterkron_fine_step_codes_are_unbounded():
    # a fine step: codes far beyond any b-bit grid, still equal to the oracle's
    c = synth.spectral(96, 80, config=2)
    _, UA = dense.prepare(c["A"], 0.01)
    _, UB = dense.prepare(c["B"], 0.01)
    Zg = check_fp64(c["W"], UA, UB, 1e-3 * transformed_rms(c["W"], UA, UB), "waterkron fine step")
    assert np.abs(Zg).max() > 1000


def check_fp32_block(W, UA, UB, alpha, beta, Zg, Vg, Ad, Bd, label):
    Zo, Vo, Yo, _ = o3.solve(W, UA, UB, beta, None, alpha=alpha)
    Z32, V32 = o3.solve(W, UA, UB, beta, None, alpha=alpha, dtype=np.float32)[:2]
    Yf = o3.solve(W, UA, UB, beta, None, alpha=alpha, force=Zg.astype(np.int32))[2]
    viol, near = compare.trajectory_violations(Zg, Yf, None, 1e-4)
    Yf32 = o3.solve(W, UA, UB, beta, None, alpha=alpha, force=Z32.astype(np.int32))[2]
    viol32, near32 = compare.trajectory_violations(Z32, Yf32, None, 1e-4)
    roots = compare.mismatch_roots(Zg != Zo)
    far = int(np.sum(roots & (compare.tie_distance(Yo) >= 1e-4)))
    mis, floor = compare.mismatch_fraction(Zg, Zo), compare.mismatch_fraction(Z32, Zo)
    loss = lambda V: dense.proxy_loss(W, V, Ad, Bd)
    lg, lo, l32 = loss(Vg), loss(Vo), loss(V32.astype(np.float64))
    rel, rel_floor = compare.rel_diff(lg, lo), compare.rel_diff(l32, lo)
    say(label, f"fp32: violations={viol} near={near} (oracle fp32 loop {viol32} / {near32}) "
               f"mismatch={mis:.3e} (oracle fp32 floor {floor:.3e}) "
               f"far roots={far} loss rel={rel:.3e} (floor {rel_floor:.3e}) entropy={dense.empirical_entropy(Zg):.3f}")
    assert viol == 0 and far == 0 and viol32 == 0
    assert near <= 4 * max(near32, 2)
    assert near > 0 or mis <= 1e-3
    assert rel <= 1e-3 or rel <= 4 * rel_floor
    return lg


def test_waterkron_fp32_spectral_256():
    c = synth.spectral()
    Ad, UA = dense.prepare(c["A"], 0.01)
    Bd, UB = dense.prepare(c["B"], 0.01)
    W32, UA32, UB32 = (x.astype(np.float32) for x in (c["W"], UA, UB))
    step = 0.5 * transformed_rms(c["W"], UA, UB)
    alpha, beta = gpu_scales(up(UA32, np.float32), up(UB32, np.float32), step, 256)
    Zg, Vg = gpu_waterkron(up(W32, np.float32), up(UA32, np.float32), up(UB32, np.float32), alpha, beta)
    a64, b64 = (t.cpu().numpy().astype(np.float64) for t in (alpha, beta))
    check_fp32_block(W32.astype(np.float64), UA32.astype(np.float64), UB32.astype(np.float64), a64, b64,
                     Zg.cpu().numpy(), Vg.cpu().numpy().astype(np.float64), Ad, Bd, "waterkron spectral 256")


@pytest.mark.timeout(300)
def test_waterkron_llm_4096_fp32():
    # The 4096 x 4096 layer of the main workload, WaterKron steps at one unit of
    # the transformed spread: full-size parity, the loss identity, the entropy.
    c = synth.llm(4096, 4096, 2, config=3)
    W = up(c["W"], np.float32)
    A, B = pipeline.factor(up(c["act"], np.float32)), pipeline.factor(up(c["grad"], np.float32))
    UA, _, _ = pipeline.prepare(A, 0.01)
    UB, _, _ = pipeline.prepare(B, 0.01)
    dA = torch.diagonal(UA).cpu().numpy().astype(np.float64)
    dB = torch.diagonal(UB).cpu().numpy().astype(np.float64)
    Wh = c["W"].astype(np.float32).astype(np.float64)
    step = float(np.sqrt(np.mean((Wh / np.outer(dB, dA)) ** 2)))
    alpha, beta = gpu_scales(UA, UB, step, 4096)
    lo = torch.zeros(1, dtype=torch.float64, device=DEV)
    Zg, Vg = gpu_waterkron(W, UA, UB, alpha, beta, loss=lo)
    trace = pipeline.loss(W, Vg, A, B, 0.01).item()
    rel_id = abs(lo.item() - trace) / trace
    hr = trace / (4096 * 4096 * step ** 2 / 12)
    say("waterkron llm 4096", f"solver loss {lo.item():.6e} kron_loss {trace:.6e} rel {rel_id:.2e}; "
                              f"loss / (m n step^2 / 12) = {hr:.3f}")
    assert rel_id <= 1e-4
    host = lambda t: t.cpu().numpy().astype(np.float64)
    Ad = dense.damp(host(A), 0.01)
    Bd = dense.damp(host(B), 0.01)
    check_fp32_block(Wh, host(UA), host(UB), host(alpha), host(beta), Zg.cpu().numpy(), host(Vg), Ad, Bd,
                     "waterkron llm 4096")
