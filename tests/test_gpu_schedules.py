"""GPU parity of the two schedules of the two-sided solver.

kron_quantize runs the recursion's leaves as one persistent launch per chunk of
tile-diagonals (each tile polls the outputs of its neighbours);
kron_quantize_per_diagonal launches one kernel per tile-diagonal.  Both run the
same operations in the same order, so codes, V and loss must be equal bit for
bit, whatever order the workgroups run the tasks in (FastKron page, section
2.3: the tiles of one tile-diagonal are independent).  The persistent solver is
also checked against the oracle on the 32 x 32 fp64 problem (literal Kronecker
GPTQ) and, in fp64, against the C left-looking loop up to the 1e-9 tie rule.
Shapes span one tile, ragged edges, several chunks and recursion levels, n > m,
and the 4096 x 4096, 1024 x 4096, 14336 x 4096 and 4096 x 14336 workloads;
kron_quantize runs twice on one workspace (its hand-over state is reset per
call).
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


def both(W, UA, UB, s, bits, per_row, ws=None):
    """kron_quantize_per_diagonal, then kron_quantize twice, on the same workspace."""
    m, n = W.shape
    if ws is None:
        ws = kq.workspace(kq.KQ_OP_QUANTIZE, W.dtype, m, n)
    outs = []
    for per_diagonal in (True, False, False):
        codes = torch.full((m, n), 99, dtype=torch.int8, device=DEV)
        V = torch.full_like(W, float("nan"))
        loss = torch.zeros(1, dtype=torch.float64, device=DEV)
        kq.kron_quantize(W, UA, UB, bits, per_row, s, codes, V, ws, loss=loss, per_diagonal=per_diagonal)
        torch.cuda.synchronize()
        outs.append((codes.cpu().numpy(), V.cpu().numpy(), float(loss.item())))
    return outs


def assert_same(outs, label):
    (z0, v0, l0) = outs[0]
    for z, v, l in outs[1:]:
        assert np.array_equal(z, z0), f"{label}: codes differ on {np.count_nonzero(z != z0)} entries"
        assert np.array_equal(v.view(np.uint8), v0.view(np.uint8)), f"{label}: V differs"
        assert l == l0, f"{label}: loss {l} vs {l0}"


def oracle_problem(W, A, B, bits, per_row):
    _, UA = dense.prepare(A, 0.01)
    _, UB = dense.prepare(B, 0.01)
    return UA, UB, dense.scales(W, bits, per_row)


def test_tiny_fp64_matches_literal_kronecker_gptq():
    c = synth.tiny()
    A = dense.factor_accumulate(c["act"], alpha=1 / 256)
    B = dense.factor_accumulate(c["grad"], alpha=1 / 256)
    Ad, UA = dense.prepare(A, 0.01)
    Bd, UB = dense.prepare(B, 0.01)
    s = dense.scales(c["W"], 4, False)
    say("schedules tiny 32x32 fp64")
    outs = both(up(c["W"], np.float64), up(UA, np.float64), up(UB, np.float64), up(s, np.float64), 4, False)
    assert_same(outs, "tiny")
    Z1, _, _ = dense.vectorized_kron_gptq(c["W"], Ad, Bd, s, 4)
    assert np.array_equal(outs[1][0], Z1)


@pytest.mark.parametrize("m,n", [(1, 1), (1, 200), (200, 1), (32, 32), (33, 65), (100, 300), (300, 100), (520, 610)])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_ragged_equals_launch_form(m, n, dtype):
    c = synth.spectral(m, n, config=60 + m % 7)
    UA, UB, s = oracle_problem(c["W"], c["A"], c["B"], 3, True)
    say("schedules", (m, n), np.dtype(dtype).name)
    outs = both(up(c["W"], dtype), up(UA, dtype), up(UB, dtype), up(s, dtype), 3, True)
    assert_same(outs, f"{m}x{n}")
    if dtype == np.float64 and m * n <= 520 * 610:
        run = lambda f: o3.solve(c["W"], UA, UB, s, 3, force=f)[0::2]
        ok, _, info = compare.codes_equal_up_to_ties(outs[1][0], run)
        assert ok, info


def test_per_tensor_scale_and_spectral_256():
    c = synth.spectral()
    UA, UB, s = oracle_problem(c["W"], c["A"], c["B"], 4, False)
    for dtype in (np.float32, np.float64):
        say("schedules spectral 256 per-tensor", np.dtype(dtype).name)
        assert_same(both(up(c["W"], dtype), up(UA, dtype), up(UB, dtype), up(s, dtype), 4, False), "256")


@pytest.mark.parametrize("m,n,bits", [(4096, 4096, 2), (1024, 4096, 3), (2048, 1536, 2), (14336, 4096, 3), (4096, 14336, 2)])
def test_llm_workloads_equal_launch_form(m, n, bits):
    c = synth.llm(m, n, bits, config=3)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    W = f32(c["W"])
    UA, _, _ = pipeline.prepare(pipeline.factor(f32(c["act"])), c["damp"])
    UB, _, _ = pipeline.prepare(pipeline.factor(f32(c["grad"])), c["damp"])
    s = torch.empty(m, dtype=torch.float32, device=DEV)
    kq.kron_row_scales(W, bits, True, s)
    say("schedules llm", (m, n))
    outs = both(W, UA, UB, s, bits, True)
    assert_same(outs, f"llm {m}x{n}")
    assert not np.isnan(outs[1][1]).any()


def test_bounded_wait_ends_the_launch(monkeypatch):
    """Every wait of the persistent solver is bounded.  With the bound forced to
    zero polls from the host (KQ_CHUNK_SPIN_LIMIT=0), a wait that is not
    satisfied at its first poll gives up and raises the abort word: the launch
    must still drain (the call returns) and the tiles swept after the abort
    store NaN in V.  The next call, with the default bound, is exact again on the
    same workspace (its hand-over state is reset per call)."""
    m = n = 512
    c = synth.spectral(m, n, config=71)
    UA, UB, s = oracle_problem(c["W"], c["A"], c["B"], 3, True)
    W, UAt, UBt, st = (up(x, np.float32) for x in (c["W"], UA, UB, s))
    ws = kq.workspace(kq.KQ_OP_QUANTIZE, W.dtype, m, n)
    codes = torch.empty((m, n), dtype=torch.int8, device=DEV)
    V = torch.empty_like(W)
    say("schedules forced abort", (m, n))
    monkeypatch.setenv("KQ_CHUNK_SPIN_LIMIT", "0")
    kq.kron_quantize(W, UAt, UBt, 3, True, st, codes, V, ws)
    torch.cuda.synchronize()
    assert torch.isnan(V).any(), "no wait gave up with a zero bound"
    monkeypatch.delenv("KQ_CHUNK_SPIN_LIMIT")
    outs = both(W, UAt, UBt, st, 3, True, ws)
    assert_same(outs, "after a forced abort")
    assert not np.isnan(outs[1][1]).any()
