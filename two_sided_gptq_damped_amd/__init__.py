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
            "kron_quantize", "kron_loss", "kron_status_string", "kron_last_error", "kron_abi_version")


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
    _check(library().kron_factor_accumulate(_dtype_code(X), rows, dim, _ptr(X), _ld(X), _ptr(S), _ld(S),
                                            float(alpha), float(beta), _stream(X.device)))
    return S


def kron_prepare(A: torch.Tensor, damp_rel: float, U: torch.Tensor, ws: torch.Tensor,
                 trace_out: torch.Tensor | None = None, lambda_out: torch.Tensor | None = None,
                 info: torch.Tensor | None = None) -> torch.Tensor:
    """U upper with U^T U = (A + damp_rel tr(A)/d I)^{-1}.  info=None waits and raises on failure."""
    d = A.shape[0]
    _check(library().kron_prepare(_dtype_code(A), d, _ptr(A), _ld(A), float(damp_rel), _ptr(U), _ld(U),
                                  _ptr(trace_out), _ptr(lambda_out), _ptr(info), _ptr(ws), ws.numel(),
                                  _stream(A.device)))
    return U


def kron_row_scales(W: torch.Tensor, bits: int, per_row: bool, scales: torch.Tensor) -> torch.Tensor:
    m, n = W.shape
    _check(library().kron_row_scales(_dtype_code(W), m, n, _ptr(W), _ld(W), int(bits), int(bool(per_row)),
                                     _ptr(scales), _stream(W.device)))
    return scales


def kron_quantize(W: torch.Tensor, U_A: torch.Tensor, U_B: torch.Tensor | None, bits: int, per_row: bool,
                  scales: torch.Tensor, codes: torch.Tensor, V: torch.Tensor, ws: torch.Tensor,
                  loss: torch.Tensor | None = None):
    """Two-sided GPTQ of W (m x n); U_B None means B = I.  Writes codes (int8) and V,
    and, if given, loss[0] (fp64) = the proxy loss of V from the rounding errors."""
    m, n = W.shape
    if loss is not None and (loss.dtype != torch.float64 or loss.numel() < 1):
        raise ValueError("kron_quantize: loss must be a float64 tensor with at least one element")
    q = _Quantizer(int(bits), int(bool(per_row)), scales.data_ptr())
    ldb = _ld(U_B) if U_B is not None else 0
    _check(library().kron_quantize(_dtype_code(W), m, n, _ptr(W), _ld(W), _ptr(U_A), _ld(U_A), _ptr(U_B), ldb,
                                   ctypes.byref(q), _ptr(codes), _ld(codes), _ptr(V), _ld(V), _ptr(loss), _ptr(ws),
                                   ws.numel(), _stream(W.device)))
    return codes, V


def kron_loss(W: torch.Tensor, V: torch.Tensor, A: torch.Tensor, B: torch.Tensor | None, damp_rel: float,
              loss_out: torch.Tensor, ws: torch.Tensor) -> torch.Tensor:
    """loss_out[0] = tr(B_d (V - W) A_d (V - W)^T) in fp64; B None means B = I."""
    m, n = W.shape
    ldb = _ld(B) if B is not None else 0
    _check(library().kron_loss(_dtype_code(W), m, n, _ptr(W), _ld(W), _ptr(V), _ld(V), _ptr(A), _ld(A), _ptr(B), ldb,
                               float(damp_rel), _ptr(loss_out), _ptr(ws), ws.numel(), _stream(W.device)))
    return loss_out


def kron_abi_version() -> int:
    return int(library().kron_abi_version())
