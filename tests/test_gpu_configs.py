"""GPU parity at the full workload sizes (LLM layer shapes), through the C ABI.

The whole path runs on the GPU exactly as the benchmark runs it: factor
accumulation from the synthetic activation / gradient rows, damped factor
preparation, per-row scales, the solver.  The oracle then solves the same
problem (the GPU's own fp32/fp64 factors and scales, promoted to fp64):
  * fp32: proxy-loss relative error <= 1e-3 against the unforced oracle, and the
    codes checked along the GPU's own trajectory: the oracle is re-run with every
    code imposed from the GPU, and each GPU code must be clamp(rne(y)) of the
    exact pre-rounding value y that the earlier codes imply, except within 1e-4
    grid units of a rounding boundary (the oracle's own fp32 loop stays within
    1.1e-5 grid units of its fp64 loop on the 4096 x 4096 layer until its first
    near-tie flip).  A near-tie decision that goes the other way in single
    precision changes the entries it feeds, so the plain mismatch fraction
    against the unforced oracle may exceed 1e-3 only when such a branch point
    exists (the oracle's own fp32 loop differs from its fp64 loop on 5.5% of the
    4096 x 4096 layer that way);
  * fp64: codes equal except at oracle pre-rounding values within 1e-9 grid
    units of a midpoint.
Where the full matrix is too large for the CPU oracle to finish in seconds the
comparison uses a leading block: by the componentwise order of the updates the
top-left k1 x k2 block of the codes depends only on W[:k1, :k2],
U_A[:k2, :k2], U_B[:k1, :k1] and the first k1 scales (scales are taken from the
full rows), so the oracle solves that block alone.  Its proxy loss uses the
factors the block problem implies, inv(U^T U) of the leading blocks.
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


def gpu_layer(c, dtype, two_sided=True, rows=None):
    """Factor, prepare, scales and quantize on the GPU; numpy copies of everything."""
    tdt = torch.float64 if dtype == np.float64 else torch.float32
    W = up(c["W"], dtype)
    act, grad = up(c["act"], dtype), up(c["grad"], dtype)
    m, n = W.shape
    A = torch.empty(n, n, dtype=tdt, device=DEV)
    kq.kron_factor_accumulate(act, A, 1.0 / act.shape[0], 0.0)
    UA, trA, _ = pipeline.prepare(A, c["damp"])
    B = UB = trB = None
    if two_sided:
        B = torch.empty(m, m, dtype=tdt, device=DEV)
        kq.kron_factor_accumulate(grad, B, 1.0 / grad.shape[0], 0.0)
        UB, trB, _ = pipeline.prepare(B, c["damp"])
    codes, V, s = pipeline.quantize(W, UA, UB, c["bits"], True)
    torch.cuda.synchronize()
    host = lambda t: None if t is None else t.cpu().numpy().astype(np.float64)
    return dict(W=host(W), A=host(A), B=host(B), UA=host(UA), UB=host(UB), s=host(s),
                Z=codes.cpu().numpy(), V=host(V), trA=trA.item(),
                trB=None if trB is None else trB.item())


def block_factor(U):
    """inv(U^T U) for an upper-triangular leading block U (fp64)."""
    Ui = np.linalg.inv(U)
    return Ui @ Ui.T


def compare_fp32(g, bits, label, k1=None, k2=None, damp=0.01):
    m, n = g["W"].shape
    k1 = m if k1 is None else k1
    k2 = n if k2 is None else k2
    W = g["W"][:k1, :k2]
    UA = g["UA"][:k2, :k2]
    UB = None if g["UB"] is None else g["UB"][:k1, :k1]
    s = g["s"][:k1]
    Zo, Vo, _, _ = o3.solve(W, UA, UB, s, bits)
    Zg, Vg = g["Z"][:k1, :k2], g["V"][:k1, :k2]
    mis = compare.mismatch_fraction(Zg, Zo)
    Yf = o3.solve(W, UA, UB, s, bits, force=Zg.astype(np.int32))[2]
    viol, near = compare.trajectory_violations(Zg, Yf, bits, 1e-4)
    if k1 == m and k2 == n:
        Ad = dense.damp(g["A"], damp)
        Bd = np.eye(m) if g["B"] is None else dense.damp(g["B"], damp)
    else:
        Ad = block_factor(UA)
        Bd = np.eye(k1) if UB is None else block_factor(UB)
    lg = dense.proxy_loss(W, Vg, Ad, Bd)
    lo = dense.proxy_loss(W, Vo, Ad, Bd)
    rel = compare.rel_diff(lg, lo)
    say(label, f"block {k1}x{k2}: trajectory violations={viol} near-tie branches={near} "
               f"mismatch vs unforced={mis:.3e} loss_gpu={lg:.6e} loss_oracle={lo:.6e} rel={rel:.3e}")
    assert viol == 0, label
    assert rel <= 1e-3, label
    assert mis <= 1e-3 or near > 0, label


def compare_fp64(g, bits, label, k1, k2):
    W = g["W"][:k1, :k2]
    UA = g["UA"][:k2, :k2]
    UB = None if g["UB"] is None else g["UB"][:k1, :k1]
    s = g["s"][:k1]
    run = lambda f: o3.solve(W, UA, UB, s, bits, force=f)[0::2]
    ok, nforced, info = compare.codes_equal_up_to_ties(g["Z"][:k1, :k2], run)
    say(label, f"fp64 block {k1}x{k2}: equal={ok} forced={nforced}")
    assert ok, f"{label}: {info}"


# ----------------------------------------- several recursion levels, fp64, full

@pytest.mark.parametrize("m,n,two_sided", [(512, 512, True), (640, 384, True), (384, 640, False),
                                           (1000, 300, True), (260, 900, True)])
def test_multilevel_fp64_full(m, n, two_sided):
    say("multilevel", m, n, "two-sided" if two_sided else "one-sided")
    c = synth.llm(m, n, 3, config=4, rows=1024)
    g = gpu_layer(c, np.float64, two_sided)
    compare_fp64(g, 3, f"multilevel {m}x{n}", m, n)


# ------------------------------------------------------ 4096 x 4096, 2-bit

@pytest.fixture(scope="module")
def layer_4096():
    return synth.llm(4096, 4096, 2, config=3)


def test_llm_4096_fp32_full(layer_4096):
    say("llm 4096x4096 fp32")
    g = gpu_layer(layer_4096, np.float32)
    compare_fp32(g, 2, "llm 4096x4096 fp32")


def test_llm_4096_fp64_corner_512(layer_4096):
    say("llm 4096x4096 fp64")
    g = gpu_layer(layer_4096, np.float64)
    compare_fp64(g, 2, "llm 4096x4096", 512, 512)
    # a second block away from the origin is not a sub-problem; the leading
    # row strip is (all columns)
    compare_fp64(g, 2, "llm 4096x4096 strip", 96, 4096)


# ------------------------------------------- GQA and gate/up shapes, 3-bit

def test_llm_1024x4096_fp32_full():
    say("llm 1024x4096 fp32")
    c = synth.llm(1024, 4096, 3, config=4)
    g = gpu_layer(c, np.float32)
    compare_fp32(g, 3, "llm 1024x4096 fp32")
    g1 = gpu_layer(c, np.float32, two_sided=False)
    compare_fp32(g1, 3, "llm 1024x4096 fp32 one-sided")


def test_llm_14336x4096_fp32_strip():
    say("llm 14336x4096 fp32")
    c = synth.llm(14336, 4096, 3, config=4)
    g = gpu_layer(c, np.float32)
    compare_fp32(g, 3, "llm 14336x4096 fp32", k1=1536)
    g1 = gpu_layer(c, np.float32, two_sided=False)
    compare_fp32(g1, 3, "llm 14336x4096 fp32 one-sided", k1=1536)


# ---------------------------------------- Llama-3-8B-shaped block, 2-bit

def test_block_sublayers_fp32_and_sensitivity():
    scores = {}
    for i in range(len(synth.BLOCK_SUBLAYERS)):
        c = synth.block_sublayer(i)
        name = synth.BLOCK_SUBLAYERS[i][0]
        say("block", name, c["W"].shape)
        g = gpu_layer(c, np.float32)
        m, n = c["W"].shape
        compare_fp32(g, 2, f"block.{name}", k1=min(m, 1024), k2=min(n, 1024))
        scores[name] = g["trA"] * g["trB"]
        # sensitivity tr(A) tr(B) of the undamped factors, against fp64 sample products
        trA = np.einsum("ij,ij->", c["act"], c["act"]) / c["act"].shape[0]
        trB = np.einsum("ij,ij->", c["grad"], c["grad"]) / c["grad"].shape[0]
        assert abs(scores[name] - trA * trB) <= 1e-5 * trA * trB
    # q, k, v share one input factor, gate and up another
    say("scores", {k: f"{v:.4e}" for k, v in scores.items()})
