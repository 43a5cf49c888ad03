"""Host-only checks of the C ABI: the library loads without a GPU, exports every
function include/kronq.h declares, sizes workspaces, and rejects bad arguments
before anything is enqueued (no HIP call is made on these paths)."""
import ctypes
import os
import re

import pytest

import two_sided_gptq_damped_amd as kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "kronq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kron_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for fn in ("kron_factor_accumulate", "kron_prepare", "kron_quantize", "kron_loss"):
        assert fn in names
    assert set(names) == set(kq.EXPORTED)


def test_library_loads_and_exports_every_declared_symbol():
    lib = kq.library()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert kq.kron_abi_version() == 4
    assert lib.kron_status_string(2) == b"factor not positive definite"


def test_workspace_sizes():
    lib = kq.library()
    q32 = lib.kron_workspace_bytes(kq.KQ_OP_QUANTIZE, kq.KQ_F32, 4096, 4096)
    q64 = lib.kron_workspace_bytes(kq.KQ_OP_QUANTIZE, kq.KQ_F64, 4096, 4096)
    # two factors plus three m x n buffers, at least
    # the loss scratch (fp64) and the chunk solver's flag words (int32) do not scale with the element size
    assert q32 >= 5 * 4096 * 4096 * 4 and q64 >= 2 * q32 - (1 << 18)
    assert lib.kron_workspace_bytes(kq.KQ_OP_QUANTIZE, kq.KQ_F32, 100, 70) >= 5 * 128 * 128 * 4
    assert lib.kron_workspace_bytes(kq.KQ_OP_PREPARE, kq.KQ_F32, 4096, 0) >= 2 * 4096 * 4096 * 8
    assert lib.kron_workspace_bytes(kq.KQ_OP_LOSS, kq.KQ_F32, 64, 64) > 0
    assert lib.kron_workspace_bytes(kq.KQ_OP_FACTOR, kq.KQ_F32, 64, 64) == 0
    assert lib.kron_workspace_bytes(kq.KQ_OP_QUANTIZE, 7, 64, 64) == 0
    assert lib.kron_workspace_bytes(kq.KQ_OP_QUANTIZE, kq.KQ_F32, -1, 64) == 0
    assert lib.kron_workspace_bytes(kq.KQ_OP_QUANTIZE, kq.KQ_F32, 1 << 17, 64) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def q(bits=3, per_row=1, scales=FAKE):
    return ctypes.byref(kq._Quantizer(bits, per_row, scales.value if scales else None))


@pytest.mark.parametrize("args,status", [
    (dict(dtype=5), 1),
    (dict(m=-1), 1),
    (dict(W=None), 1),
    (dict(UA=None), 1),
    (dict(codes=None), 1),
    (dict(V=None), 1),
    (dict(ldw=10), 1),
    (dict(lda=10), 1),
    (dict(ldb=10), 1),
    (dict(ldc=10), 1),
    (dict(q=None), 1),
    (dict(bits=1), 1),
    (dict(bits=9), 1),
    (dict(per_row=2), 1),
    (dict(scales=None), 1),
    (dict(ws=None), 3),
    (dict(ws_bytes=1024), 3),
    (dict(m=1 << 17), 1),
])
def test_quantize_rejects_bad_arguments(args, status):
    lib = kq.library()
    a = dict(dtype=kq.KQ_F32, m=64, n=64, W=FAKE, ldw=64, UA=FAKE, lda=64, UB=FAKE, ldb=64, bits=3, per_row=1,
             scales=FAKE, codes=FAKE, ldc=64, V=FAKE, ldv=64, loss=None, ws=FAKE, ws_bytes=1 << 40, q=True)
    a.update(args)
    qq = q(a["bits"], a["per_row"], a["scales"]) if a["q"] else None
    rc = lib.kron_quantize(a["dtype"], a["m"], a["n"], a["W"], a["ldw"], a["UA"], a["lda"], a["UB"], a["ldb"], qq,
                           a["codes"], a["ldc"], a["V"], a["ldv"], a["loss"], a["ws"], a["ws_bytes"], None)
    assert rc == status
    assert lib.kron_last_error() != b""


def test_quantize_empty_is_a_no_op():
    lib = kq.library()
    assert lib.kron_quantize(kq.KQ_F32, 0, 64, None, 64, None, 64, None, 0, q(), None, 64, None, 64, None, None, 0,
                             None) == 0
    assert lib.kron_quantize(kq.KQ_F64, 64, 0, None, 0, None, 0, None, 64, q(), None, 0, None, 0, None, None, 0,
                             None) == 0
    # an empty matrix has no loss to report
    assert lib.kron_quantize(kq.KQ_F64, 64, 0, None, 0, None, 0, None, 64, q(), None, 0, None, 0, FAKE, None, 0,
                             None) == 1


def test_workspace_alignment_is_checked():
    lib = kq.library()
    rc = lib.kron_quantize(kq.KQ_F32, 64, 64, FAKE, 64, FAKE, 64, None, 0, q(), FAKE, 64, FAKE, 64, None,
                           ctypes.c_void_p(0x1008), 1 << 40, None)
    assert rc == 3 and b"aligned" in lib.kron_last_error()


def test_prepare_factor_loss_scales_reject_bad_arguments():
    lib = kq.library()
    assert lib.kron_prepare(kq.KQ_F32, 0, FAKE, 1, 0.01, FAKE, 1, None, None, None, FAKE, 1 << 40, None) == 1
    assert lib.kron_prepare(kq.KQ_F32, 64, None, 64, 0.01, FAKE, 64, None, None, None, FAKE, 1 << 40, None) == 1
    assert lib.kron_prepare(kq.KQ_F32, 64, FAKE, 32, 0.01, FAKE, 64, None, None, None, FAKE, 1 << 40, None) == 1
    assert lib.kron_prepare(kq.KQ_F32, 64, FAKE, 64, -1.0, FAKE, 64, None, None, None, FAKE, 1 << 40, None) == 1
    assert lib.kron_prepare(kq.KQ_F32, 64, FAKE, 64, float("nan"), FAKE, 64, None, None, None, FAKE, 1 << 40,
                            None) == 1
    assert lib.kron_prepare(kq.KQ_F32, 64, FAKE, 64, 0.01, FAKE, 64, None, None, None, FAKE, 16, None) == 3
    assert lib.kron_factor_accumulate(kq.KQ_F32, 10, 64, None, 64, FAKE, 64, 1.0, 0.0, None) == 1
    assert lib.kron_factor_accumulate(kq.KQ_F32, 10, 64, FAKE, 63, FAKE, 64, 1.0, 0.0, None) == 1
    assert lib.kron_factor_accumulate(kq.KQ_F32, 10, 64, FAKE, 64, FAKE, 64, float("inf"), 0.0, None) == 1
    assert lib.kron_factor_accumulate(kq.KQ_F32, 10, 0, None, 0, None, 0, 1.0, 0.0, None) == 0
    assert lib.kron_loss(kq.KQ_F64, 8, 8, FAKE, 8, None, 8, FAKE, 8, None, 0, 0.0, FAKE, FAKE, 1 << 40, None) == 1
    assert lib.kron_loss(kq.KQ_F64, 8, 8, FAKE, 8, FAKE, 8, FAKE, 8, FAKE, 4, 0.0, FAKE, FAKE, 1 << 40, None) == 1
    assert lib.kron_loss(kq.KQ_F64, 8, 8, FAKE, 8, FAKE, 8, FAKE, 8, None, 0, 0.0, FAKE, FAKE, 8, None) == 3
    assert lib.kron_row_scales(kq.KQ_F32, 8, 8, FAKE, 8, 1, 1, FAKE, None) == 1
    assert lib.kron_row_scales(kq.KQ_F32, 8, 8, FAKE, 8, 4, 3, FAKE, None) == 1
    assert lib.kron_row_scales(kq.KQ_F32, 8, 8, None, 8, 4, 1, FAKE, None) == 1


def test_binding_rejects_mismatched_arguments():
    # The C entry points see raw pointers only, so the binding checks element
    # type, device and shape of every tensor before the call (CPU tensors here:
    # each check fails before the library is reached).
    torch = pytest.importorskip("torch")
    m, n = 6, 5
    W = torch.zeros(m, n)
    UA, UB = torch.zeros(n, n), torch.zeros(m, m)
    s, codes, V = torch.ones(m), torch.zeros(m, n, dtype=torch.int8), torch.zeros(m, n)
    ws = torch.zeros(256, dtype=torch.uint8)
    bad = [
        dict(U_A=UA.double()), dict(U_B=UB[:4, :4]), dict(scales=s.double()), dict(scales=s[:3]),
        dict(codes=codes.int()), dict(V=V.double()), dict(ws=ws.float()),
        dict(loss=torch.zeros(1)), dict(codes=torch.zeros(n, m, dtype=torch.int8)),
    ]
    for change in bad:
        args = dict(W=W, U_A=UA, U_B=UB, bits=3, per_row=True, scales=s, codes=codes, V=V, ws=ws, loss=None)
        args.update(change)
        with pytest.raises(ValueError):
            kq.kron_quantize(**args)
    with pytest.raises(ValueError):
        kq.kron_prepare(UA, 0.01, UA.double(), ws)
    with pytest.raises(ValueError):
        kq.kron_prepare(UA, 0.01, UA, ws, info=torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError):
        kq.kron_loss(W, V, UA, UB.double(), 0.01, torch.zeros(1, dtype=torch.float64), ws)
    with pytest.raises(ValueError):
        kq.kron_factor_accumulate(W, torch.zeros(n, n, dtype=torch.float64), 1.0, 0.0)


def test_noalloc_rejects_before_any_device_call():
    lib = kq.library()
    # too large for the fixed scratch array: KQ_ERR_WORKSPACE, nothing enqueued
    need = lib.kron_workspace_bytes(kq.KQ_OP_QUANTIZE, kq.KQ_F32, 4096, 4096)
    assert need > kq.NOALLOC_SCRATCH_BYTES
    assert lib.kron_quantize_noalloc(kq.KQ_F32, 4096, 4096, FAKE, 4096, FAKE, 4096, FAKE, 4096, q(), FAKE, 4096,
                                     FAKE, 4096, None, None) == 3
    assert b"scratch" in lib.kron_last_error()
    # the argument checks of kron_quantize
    assert lib.kron_quantize_noalloc(kq.KQ_F32, 64, 64, None, 64, FAKE, 64, FAKE, 64, q(), FAKE, 64,
                                     FAKE, 64, None, None) == 1
    assert lib.kron_quantize_noalloc(kq.KQ_F32, 64, 64, FAKE, 64, FAKE, 64, FAKE, 64, q(bits=9), FAKE, 64,
                                     FAKE, 64, None, None) == 1
    assert lib.kron_quantize_noalloc(kq.KQ_F32, 0, 64, None, 64, None, 64, None, 0, q(), None, 64,
                                     None, 64, None, None) == 0


def test_waterkron_entry_points_validate_on_the_host():
    lib = kq.library()
    F = FAKE
    # kron_waterkron_scales: step must be positive and finite; null pointers; sizes
    assert lib.kron_waterkron_scales(kq.KQ_F32, 8, 8, F, 8, None, 0, 0.0, F, F, None) == 1
    assert lib.kron_waterkron_scales(kq.KQ_F32, 8, 8, F, 8, None, 0, float("inf"), F, F, None) == 1
    assert lib.kron_waterkron_scales(kq.KQ_F32, 8, 8, None, 8, None, 0, 1.0, F, F, None) == 1
    assert lib.kron_waterkron_scales(kq.KQ_F32, 0, 8, F, 8, None, 0, 1.0, F, F, None) == 1
    assert lib.kron_waterkron_scales(kq.KQ_F32, 8, 8, F, 8, F, 4, 1.0, F, F, None) == 1
    # kron_quantize_waterkron: null scales, leading dimensions, workspace
    args = [kq.KQ_F64, 8, 8, F, 8, F, 8, F, 8, F, F, F, 8, F, 8, None, F, 1 << 40, None]
    assert lib.kron_quantize_waterkron(*args[:9], None, *args[10:]) == 1
    assert lib.kron_quantize_waterkron(*args[:12], 4, *args[13:]) == 1
    assert lib.kron_quantize_waterkron(*args[:17], 16, None) == 3
    assert lib.kron_quantize_waterkron(kq.KQ_F64, 0, 8, None, 8, None, 8, None, 0, None, None, None, 8, None, 8,
                                       None, None, 0, None) == 0


def test_kronecker_entry_point_validates_on_the_host():
    lib = kq.library()
    F = FAKE
    good = [kq.KQ_F32, kq.KQ_KRON_FLIPFLOP, 256, 64, 32, F, 64, F, 32, 2, 0.01, F, 64, F, 32, None, F, 1 << 40, None]
    def call(**kw):
        args = list(good)
        for i, v in kw.items():
            args[int(i[1:])] = v
        return lib.kron_factor_kronecker(*args)
    assert call(a1=2) == 1            # method
    assert call(a9=0) == 1 and call(a9=65) == 1  # iters
    assert call(a5=None) == 1         # Xa
    assert call(a6=63) == 1           # ldxa < n
    assert call(a10=-1.0) == 1        # damp_rel
    assert call(a17=16) == 3          # workspace too small
    need = lib.kron_kronecker_workspace_bytes(kq.KQ_F32, 256, 64, 32)
    assert need > 256 * 64 * 4 and lib.kron_kronecker_workspace_bytes(kq.KQ_F32, 0, 64, 32) == 0


def test_biip_entry_points_validate_on_the_host():
    lib = kq.library()
    F = FAKE
    fw = [kq.KQ_F32, 64, 48, F, 48, F, 48, F, 64, F, F, F, 48, F, 48, F, 64, F, F, F, 1 << 40, None]
    assert lib.kron_biip_forward(*fw[:9], None, *fw[10:]) == 1        # signs_n
    assert lib.kron_biip_forward(*fw[:4], 40, *fw[5:]) == 1            # ldw < n
    assert lib.kron_biip_forward(*fw[:20], 64, None) == 3              # workspace
    inv = [kq.KQ_F64, 64, 48, F, 48, F, F, F, F, F, 48, F, 1 << 40, None]
    assert lib.kron_biip_inverse(*inv[:7], None, *inv[8:]) == 1        # scale_a
    assert lib.kron_biip_inverse(*inv[:10], 40, *inv[11:]) == 1        # ldv < n
    assert lib.kron_biip_workspace_bytes(kq.KQ_F32, 64, 48) >= 2 * 64 * 64 * 4
