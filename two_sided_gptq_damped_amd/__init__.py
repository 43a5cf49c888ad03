"""Python binding of libkronq (two-sided GPTQ on MI355X / gfx950).

Argument marshalling only: each function below converts torch tensors to raw
device pointers, sizes and leading dimensions and calls the C entry point of
the same name in ``libkronq.so`` (declared in ``include/kronq.h``) on torch's
current HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  If the library has not been built, or cannot be
loaded, the first call raises ``RuntimeError``.

Build with ``python -m two_sided_gptq_damped_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkronq.so")

KQ_F32, KQ_F64 = 0, 1
KQ_OP_FACTOR, KQ_OP_PREPARE, KQ_OP_QUANTIZE, KQ_OP_LOSS = 0, 1, 2, 3
STATUS = {0: "KQ_OK", 1: "KQ_ERR_INVALID_ARG", 2: "KQ_ERR_NOT_PD", 3: "KQ_ERR_WORKSPACE",
          4: "KQ_ERR_HIP", 5: "KQ_ERR_UNSUPPORTED"}
EXPORTED = ("kron_workspace_bytes", "kron_factor_accumulate", "kron_prepare", "kron_row_scales",
            "kron_quantize", "kron_loss", "kron_status_string", "kron_last_error", "kron_abi_version",
            "kron_quantize_noalloc", "kron_waterkron_scales", "kron_quantize_waterkron",
            "kron_kronecker_workspace_bytes", "kron_factor_kronecker", "kron_biip_workspace_bytes",
            "kron_biip_forward", "kron_biip_inverse", "kron_quantize_per_diagonal")
KQ_KRON_FROBENIUS, KQ_KRON_FLIPFLOP = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # KQ_NOALLOC_SCRATCH_BYTES


class KronError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class _Quantizer(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("per_row", ctypes.c_int32), ("scales", ctypes.c_void_p)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libkronq.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkronq.so not found at {LIB_PATH}: build it with "
                           "`python -m two_sided_gptq_damped_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, dbl, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double, ctypes.c_size_t
    lib.kron_workspace_bytes.restype = sz
    lib.kron_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64]
    lib.kron_factor_accumulate.restype = ctypes.c_int
    lib.kron_factor_accumulate.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, i64, dbl, dbl, vp]
    lib.kron_prepare.restype = ctypes.c_int
    lib.kron_prepare.argtypes = [ctypes.c_int, i64, vp, i64, dbl, vp, i64, vp, vp, vp, vp, sz, vp]
    lib.kron_row_scales.restype = ctypes.c_int
    lib.kron_row_scales.argtypes = [ctypes.c_int, i64, i64, vp, i64, i32, i32, vp, vp]
    lib.kron_quantize.restype = ctypes.c_int
    lib.kron_quantize.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, i64, vp, i64,
                                  ctypes.POINTER(_Quantizer), vp, i64, vp, i64, vp, vp, sz, vp]
    lib.kron_quantize_per_diagonal.restype = ctypes.c_int
    lib.kron_quantize_per_diagonal.argtypes = lib.kron_quantize.argtypes
    lib.kron_quantize_noalloc.restype = ctypes.c_int
    lib.kron_quantize_noalloc.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, i64, vp, i64,
                                          ctypes.POINTER(_Quantizer), vp, i64, vp, i64, vp, vp]
    lib.kron_biip_workspace_bytes.restype = sz
    lib.kron_biip_workspace_bytes.argtypes = [ctypes.c_int, i64, i64]
    lib.kron_biip_forward.restype = ctypes.c_int
    lib.kron_biip_forward.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, i64, vp, i64, vp, vp, vp, i64, vp, i64, vp,
                                      i64, vp, vp, vp, sz, vp]
    lib.kron_biip_inverse.restype = ctypes.c_int
    lib.kron_biip_inverse.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, vp, vp, vp, vp, i64, vp, sz, vp]
    lib.kron_kronecker_workspace_bytes.restype = sz
    lib.kron_kronecker_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64]
    lib.kron_factor_kronecker.restype = ctypes.c_int
    lib.kron_factor_kronecker.argtypes = [ctypes.c_int, i32, i64, i64, i64, vp, i64, vp, i64, i32, dbl, vp, i64, vp,
                                          i64, vp, vp, sz, vp]
    lib.kron_waterkron_scales.restype = ctypes.c_int
    lib.kron_waterkron_scales.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, i64, dbl, vp, vp, vp]
    lib.kron_quantize_waterkron.restype = ctypes.c_int
    lib.kron_quantize_waterkron.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, i64, vp, i64, vp, vp, vp, i64, vp,
                                            i64, vp, vp, sz, vp]
    lib.kron_loss.restype = ctypes.c_int
    lib.kron_loss.argtypes = [ctypes.c_int, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, dbl, vp, vp, sz, vp]
    lib.kron_status_string.restype = ctypes.c_char_p
    lib.kron_status_string.argtypes = [ctypes.c_int]
    lib.kron_last_error.restype = ctypes.c_char_p
    lib.kron_last_error.argtypes = []
    lib.kron_abi_version.restype = ctypes.c_int32
    lib.kron_abi_version.argtypes = []
    _lib = lib
    return lib


# ------------------------------------------------------------------ marshalling

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KQ_F32
    if t.dtype == torch.float64:
        return KQ_F64
    raise TypeError(f"expected float32 or float64 tensor, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t, name: str, dtype: torch.dtype, device: torch.device, numel: int | None = None,
            shape: tuple | None = None) -> None:
    """Reject an argument whose element type, device or shape differs from what
    the C entry point will read it as (the library sees only a raw pointer)."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected a tensor on {device}, got {t.device}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: expected at least {numel} elements, got {t.numel()}")


def _ld(t: torch.Tensor) -> int:
    """Leading dimension of a row-major 2-D view (unit column stride required)."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError("expected unit stride along columns (row-major)")
    return max(t.stride(0), t.shape[1], 1)


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int) -> None:
    if status != 0:
        raise KronError(status, library().kron_last_error().decode())


def kron_workspace_bytes(op: int, dtype: torch.dtype, m: int, n: int) -> int:
    code = KQ_F64 if dtype == torch.float64 else KQ_F32
    return int(library().kron_workspace_bytes(op, code, m, n))


def workspace(op: int, dtype: torch.dtype, m: int, n: int, device="cuda") -> torch.Tensor:
    """A device byte buffer large enough for ``op`` (256-byte aligned by torch's allocator)."""
    nbytes = kron_workspace_bytes(op, dtype, m, n)
    buf = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(nbytes, 256)]


def kron_factor_accumulate(X: torch.Tensor, S: torch.Tensor, alpha: float, beta: float) -> torch.Tensor:
    """S <- beta S + alpha X^T X (X: rows x dim samples)."""
    rows, dim = X.shape
    _expect(S, "S", X.dtype, X.device, shape=(dim, dim))
    _check(library().kron_factor_accumulate(_dtype_code(X), rows, dim, _ptr(X), _ld(X), _ptr(S), _ld(S),
                                            float(alpha), float(beta), _stream(X.device)))
    return S


def kron_prepare(A: torch.Tensor, damp_rel: float, U: torch.Tensor, ws: torch.Tensor,
                 trace_out: torch.Tensor | None = None, lambda_out: torch.Tensor | None = None,
                 info: torch.Tensor | None = None) -> torch.Tensor:
    """U upper with U^T U = (A + damp_rel tr(A)/d I)^{-1}.  info=None waits and raises on failure."""
    d = A.shape[0]
    _expect(U, "U", A.dtype, A.device, shape=(d, d))
    _expect(ws, "ws", torch.uint8, A.device)
    for t, name in ((trace_out, "trace_out"), (lambda_out, "lambda_out")):
        _expect(t, name, torch.float64, A.device, 1)
    _expect(info, "info", torch.int32, A.device, 1)
    _check(library().kron_prepare(_dtype_code(A), d, _ptr(A), _ld(A), float(damp_rel), _ptr(U), _ld(U),
                                  _ptr(trace_out), _ptr(lambda_out), _ptr(info), _ptr(ws), ws.numel(),
                                  _stream(A.device)))
    return U


def kron_row_scales(W: torch.Tensor, bits: int, per_row: bool, scales: torch.Tensor) -> torch.Tensor:
    m, n = W.shape
    _expect(scales, "scales", W.dtype, W.device, m if per_row else 1)
    _check(library().kron_row_scales(_dtype_code(W), m, n, _ptr(W), _ld(W), int(bits), int(bool(per_row)),
                                     _ptr(scales), _stream(W.device)))
    return scales


def kron_quantize(W: torch.Tensor, U_A: torch.Tensor, U_B: torch.Tensor | None, bits: int, per_row: bool,
                  scales: torch.Tensor, codes: torch.Tensor, V: torch.Tensor, ws: torch.Tensor,
                  loss: torch.Tensor | None = None, per_diagonal: bool = False):
    """Two-sided GPTQ of W (m x n); U_B None means B = I.  Writes codes (int8) and V,
    and, if given, loss[0] (fp64) = the proxy loss of V from the rounding errors.
    per_diagonal: call kron_quantize_per_diagonal (the same results, the
    two-sided leaves launched one kernel per tile-diagonal)."""
    m, n = W.shape
    for t, name, shp in ((U_A, "U_A", (n, n)), (U_B, "U_B", (m, m)), (V, "V", (m, n))):
        _expect(t, name, W.dtype, W.device, shape=shp)
    _expect(scales, "scales", W.dtype, W.device, m if per_row else 1)
    _expect(codes, "codes", torch.int8, W.device, shape=(m, n))
    _expect(ws, "ws", torch.uint8, W.device)
    _expect(loss, "loss", torch.float64, W.device, 1)
    q = _Quantizer(int(bits), int(bool(per_row)), scales.data_ptr())
    ldb = _ld(U_B) if U_B is not None else 0
    fn = library().kron_quantize_per_diagonal if per_diagonal else library().kron_quantize
    _check(fn(_dtype_code(W), m, n, _ptr(W), _ld(W), _ptr(U_A), _ld(U_A), _ptr(U_B), ldb, ctypes.byref(q),
              _ptr(codes), _ld(codes), _ptr(V), _ld(V), _ptr(loss), _ptr(ws), ws.numel(), _stream(W.device)))
    return codes, V


def kron_quantize_noalloc(W: torch.Tensor, U_A: torch.Tensor, U_B: torch.Tensor | None, bits: int, per_row: bool,
                          scales: torch.Tensor, codes: torch.Tensor, V: torch.Tensor,
                          loss: torch.Tensor | None = None):
    """kron_quantize without a workspace: the library's fixed per-GPU scratch
    array is used instead (nothing is allocated; sizes that need more than
    NOALLOC_SCRATCH_BYTES raise KronError with KQ_ERR_WORKSPACE)."""
    m, n = W.shape
    for t, name, shp in ((U_A, "U_A", (n, n)), (U_B, "U_B", (m, m)), (V, "V", (m, n))):
        _expect(t, name, W.dtype, W.device, shape=shp)
    _expect(scales, "scales", W.dtype, W.device, m if per_row else 1)
    _expect(codes, "codes", torch.int8, W.device, shape=(m, n))
    _expect(loss, "loss", torch.float64, W.device, 1)
    q = _Quantizer(int(bits), int(bool(per_row)), scales.data_ptr())
    ldb = _ld(U_B) if U_B is not None else 0
    with torch.cuda.device(W.device):
        _check(library().kron_quantize_noalloc(_dtype_code(W), m, n, _ptr(W), _ld(W), _ptr(U_A), _ld(U_A), _ptr(U_B),
                                               ldb, ctypes.byref(q), _ptr(codes), _ld(codes), _ptr(V), _ld(V),
                                               _ptr(loss), _stream(W.device)))
    return codes, V


def kronecker_workspace(dtype: torch.dtype, samples: int, n: int, m: int, device="cuda") -> torch.Tensor:
    """A device byte buffer for kron_factor_kronecker (256-byte aligned)."""
    code = KQ_F64 if dtype == torch.float64 else KQ_F32
    nbytes = int(library().kron_kronecker_workspace_bytes(code, samples, n, m))
    buf = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(nbytes, 256)]


def kron_factor_kronecker(Xa: torch.Tensor, Xb: torch.Tensor, method: int, iters: int, damp_rel: float,
                          A: torch.Tensor, B: torch.Tensor, ws: torch.Tensor, info: torch.Tensor | None = None):
    """FlipFlop / Frobenius Kronecker factors A (n x n), B (m x m) from paired
    sample rows Xa (N x n) and Xb (N x m).  info=None waits and raises if a
    damped FlipFlop factor is not positive definite."""
    N, n = Xa.shape
    m = Xb.shape[1]
    if Xb.shape[0] != N:
        raise ValueError("Xa and Xb must have the same number of sample rows")
    _expect(Xb, "Xb", Xa.dtype, Xa.device)
    _expect(A, "A", Xa.dtype, Xa.device, shape=(n, n))
    _expect(B, "B", Xa.dtype, Xa.device, shape=(m, m))
    _expect(ws, "ws", torch.uint8, Xa.device)
    _expect(info, "info", torch.int32, Xa.device, 1)
    _check(library().kron_factor_kronecker(_dtype_code(Xa), int(method), N, n, m, _ptr(Xa), _ld(Xa), _ptr(Xb), _ld(Xb),
                                           int(iters), float(damp_rel), _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(info),
                                           _ptr(ws), ws.numel(), _stream(Xa.device)))
    return A, B


def biip_workspace(dtype: torch.dtype, m: int, n: int, device="cuda") -> torch.Tensor:
    """A device byte buffer for kron_biip_forward / kron_biip_inverse (256-byte aligned)."""
    code = KQ_F64 if dtype == torch.float64 else KQ_F32
    nbytes = int(library().kron_biip_workspace_bytes(code, m, n))
    buf = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(nbytes, 256)]


def kron_biip_forward(W, A, B, signs_n, signs_m, W_out, A_out, B_out, scale_a, scale_b, ws):
    """KronQ BiIP: W_out = Q_B S_B W S_A Q_A^T, A_out, B_out the matching factors;
    scale_a = diag(A)^{-1/4}, scale_b = diag(B)^{-1/4}."""
    m, n = W.shape
    for t, name, shp in ((A, "A", (n, n)), (B, "B", (m, m)), (W_out, "W_out", (m, n)), (A_out, "A_out", (n, n)),
                         (B_out, "B_out", (m, m))):
        _expect(t, name, W.dtype, W.device, shape=shp)
    _expect(signs_n, "signs_n", torch.int8, W.device, n)
    _expect(signs_m, "signs_m", torch.int8, W.device, m)
    _expect(scale_a, "scale_a", W.dtype, W.device, n)
    _expect(scale_b, "scale_b", W.dtype, W.device, m)
    _expect(ws, "ws", torch.uint8, W.device)
    _check(library().kron_biip_forward(_dtype_code(W), m, n, _ptr(W), _ld(W), _ptr(A), _ld(A), _ptr(B), _ld(B),
                                       _ptr(signs_n), _ptr(signs_m), _ptr(W_out), _ld(W_out), _ptr(A_out), _ld(A_out),
                                       _ptr(B_out), _ld(B_out), _ptr(scale_a), _ptr(scale_b), _ptr(ws), ws.numel(),
                                       _stream(W.device)))
    return W_out, A_out, B_out


def kron_biip_inverse(V2, signs_n, signs_m, scale_a, scale_b, V, ws):
    """V = S_B^{-1} Q_B^T V2 Q_A S_A^{-1} (the processed problem's result mapped back)."""
    m, n = V2.shape
    _expect(V, "V", V2.dtype, V2.device, shape=(m, n))
    _expect(signs_n, "signs_n", torch.int8, V2.device, n)
    _expect(signs_m, "signs_m", torch.int8, V2.device, m)
    _expect(scale_a, "scale_a", V2.dtype, V2.device, n)
    _expect(scale_b, "scale_b", V2.dtype, V2.device, m)
    _expect(ws, "ws", torch.uint8, V2.device)
    _check(library().kron_biip_inverse(_dtype_code(V2), m, n, _ptr(V2), _ld(V2), _ptr(signs_n), _ptr(signs_m),
                                       _ptr(scale_a), _ptr(scale_b), _ptr(V), _ld(V), _ptr(ws), ws.numel(),
                                       _stream(V2.device)))
    return V


def kron_waterkron_scales(U_A: torch.Tensor, U_B: torch.Tensor | None, step: float, alpha: torch.Tensor,
                          beta: torch.Tensor) -> tuple:
    """WaterKron scales: alpha = step * diag(U_A) (n), beta = diag(U_B) or 1 (m)."""
    n, m = U_A.shape[0], beta.numel()
    _expect(U_B, "U_B", U_A.dtype, U_A.device, shape=(m, m))
    _expect(alpha, "alpha", U_A.dtype, U_A.device, n)
    _expect(beta, "beta", U_A.dtype, U_A.device, m)
    ldb = _ld(U_B) if U_B is not None else 0
    _check(library().kron_waterkron_scales(_dtype_code(U_A), m, n, _ptr(U_A), _ld(U_A), _ptr(U_B), ldb, float(step),
                                           _ptr(alpha), _ptr(beta), _stream(U_A.device)))
    return alpha, beta


def kron_quantize_waterkron(W: torch.Tensor, U_A: torch.Tensor, U_B: torch.Tensor | None, alpha: torch.Tensor,
                            beta: torch.Tensor, codes: torch.Tensor, V: torch.Tensor, ws: torch.Tensor,
                            loss: torch.Tensor | None = None):
    """Two-sided GPTQ with per-entry steps beta_i alpha_j and unbounded int32 codes."""
    m, n = W.shape
    for t, name, shp in ((U_A, "U_A", (n, n)), (U_B, "U_B", (m, m)), (V, "V", (m, n))):
        _expect(t, name, W.dtype, W.device, shape=shp)
    _expect(alpha, "alpha", W.dtype, W.device, n)
    _expect(beta, "beta", W.dtype, W.device, m)
    _expect(codes, "codes", torch.int32, W.device, shape=(m, n))
    _expect(ws, "ws", torch.uint8, W.device)
    _expect(loss, "loss", torch.float64, W.device, 1)
    ldb = _ld(U_B) if U_B is not None else 0
    _check(library().kron_quantize_waterkron(_dtype_code(W), m, n, _ptr(W), _ld(W), _ptr(U_A), _ld(U_A), _ptr(U_B),
                                             ldb, _ptr(alpha), _ptr(beta), _ptr(codes), _ld(codes), _ptr(V), _ld(V),
                                             _ptr(loss), _ptr(ws), ws.numel(), _stream(W.device)))
    return codes, V


def kron_loss(W: torch.Tensor, V: torch.Tensor, A: torch.Tensor, B: torch.Tensor | None, damp_rel: float,
              loss_out: torch.Tensor, ws: torch.Tensor) -> torch.Tensor:
    """loss_out[0] = tr(B_d (V - W) A_d (V - W)^T) in fp64; B None means B = I."""
    m, n = W.shape
    for t, name, shp in ((V, "V", (m, n)), (A, "A", (n, n)), (B, "B", (m, m))):
        _expect(t, name, W.dtype, W.device, shape=shp)
    _expect(loss_out, "loss_out", torch.float64, W.device, 1)
    _expect(ws, "ws", torch.uint8, W.device)
    ldb = _ld(B) if B is not None else 0
    _check(library().kron_loss(_dtype_code(W), m, n, _ptr(W), _ld(W), _ptr(V), _ld(V), _ptr(A), _ld(A), _ptr(B), ldb,
                               float(damp_rel), _ptr(loss_out), _ptr(ws), ws.numel(), _stream(W.device)))
    return loss_out


def kron_abi_version() -> int:
    return int(library().kron_abi_version())
