"""kron_quantize_noalloc (for callers that cannot allocate) against kron_quantize.

Both run the same kernels on the same inputs; the no-allocation variant takes
its scratch from the library's fixed per-GPU array instead of a workspace, so
codes, V and the loss must be bitwise equal.  Two calls in a row, the second on
a smaller problem (the array keeps the first call's contents), fp32 and fp64,
two-sided and B = I.
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

DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)


def problem(m, n, dtype, seed):
    c = synth.spectral(m, n, config=seed)
    _, UA = dense.prepare(c["A"], 0.01)
    _, UB = dense.prepare(c["B"], 0.01)
    s = dense.scales(c["W"], 3, True)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a.astype(dtype))).to(DEV)
    return up(c["W"]), up(UA), up(UB), up(s)


def both(W, UA, UB, s):
    m, n = W.shape
    out = []
    for noalloc in (False, True):
        codes = torch.empty(m, n, dtype=torch.int8, device=DEV)
        V = torch.empty_like(W)
        loss = torch.zeros(1, dtype=torch.float64, device=DEV)
        if noalloc:
            kq.kron_quantize_noalloc(W, UA, UB, 3, True, s, codes, V, loss=loss)
        else:
            ws = kq.workspace(kq.KQ_OP_QUANTIZE, W.dtype, m, n)
            kq.kron_quantize(W, UA, UB, 3, True, s, codes, V, ws, loss=loss)
        out.append((codes, V, loss))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("two_sided", [True, False])
def test_noalloc_matches_workspace_entry_point(dtype, two_sided):
    for k, (m, n) in enumerate([(700, 900), (130, 70)]):  # the second call is smaller
        W, UA, UB, s = problem(m, n, dtype, 20 + k)
        say("noalloc", np.dtype(dtype).name, "two-sided" if two_sided else "B=I", (m, n))
        (c0, v0, l0), (c1, v1, l1) = both(W, UA, UB if two_sided else None, s)
        assert torch.equal(c0, c1) and torch.equal(v0, v1) and l0.item() == l1.item()


def test_noalloc_rejects_a_size_beyond_its_array():
    W = torch.zeros(4096, 4096, dtype=torch.float32, device=DEV)
    U = torch.eye(4096, dtype=torch.float32, device=DEV)
    s = torch.ones(4096, dtype=torch.float32, device=DEV)
    codes = torch.empty(4096, 4096, dtype=torch.int8, device=DEV)
    with pytest.raises(kq.KronError) as e:
        kq.kron_quantize_noalloc(W, U, U, 3, True, s, codes, torch.empty_like(W))
    assert e.value.status == 3
