"""ctypes front end of tier O3 (oracle/o3.c).  TEST INFRASTRUCTURE ONLY.

``build()`` compiles o3.c with gcc into two shared objects in this folder
(fp64 and fp32 arithmetic).  ``solve`` takes the upper factors U_A, U_B
(U^T U = A_d^{-1}), forms the normalised lower factors L~ = (U / diag(U))^T in
the run precision, and calls the C loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "o3.c")
NOT_FORCED = -(2 ** 31)
_LIBS: dict = {}


def _lib_path(tag: str) -> str:
    return os.path.join(HERE, f"liboracle_o3_{tag}.so")


def build(force: bool = True) -> None:
    """Compile o3.c (fp64 and fp32 variants).  Portable x86-64-v3 code, no fast-math."""
    for tag, real in (("f64", "double"), ("f32", "float")):
        out = _lib_path(tag)
        if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
            continue
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-ffp-contract=fast",
               "-fPIC", "-shared", f"-DREAL={real}", "-o", out + ".tmp", SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    _LIBS.clear()


def _load(tag: str):
    if tag not in _LIBS:
        path = _lib_path(tag)
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
            build(force=False)
        lib = ctypes.CDLL(path)
        fn = lib.o3_solve
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 5 + \
            [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
             ctypes.c_void_p, ctypes.c_int]
        _LIBS[tag] = fn
    return _LIBS[tag]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def lower_normalized(U: np.ndarray, dtype) -> np.ndarray:
    """L~[r][c] = U[c][r] / U[c][c] computed in ``dtype`` (IEEE division)."""
    U = np.asarray(U).astype(dtype)
    return np.ascontiguousarray((U / np.diag(U)[:, None]).T)


def solve(W, UA, UB, s, bits, dtype=np.float64, force=None, threads=0, La=None, Lb=None, alpha=None):
    """Left-looking two-sided GPTQ.  UB=None means B = I (one-sided GPTQ).

    ``s`` has length m (per row) or 1 (per tensor).  ``alpha`` (length n) adds
    column scales: entry (i, j) then has the step s_i alpha_j (WaterKron).
    bits=None leaves the codes unbounded.  ``force`` is an optional m x n int32
    array of imposed codes (NOT_FORCED elsewhere).  Precomputed La / Lb (as
    returned by ``lower_normalized``) may be passed to skip re-normalising.
    Returns (Z, V, Y fp64 pre-rounding value x/s, D errors); Z is int8 for a
    b-bit grid and int32 when unbounded.
    """
    dtype = np.dtype(dtype)
    tag = "f64" if dtype == np.float64 else "f32"
    W = np.ascontiguousarray(np.asarray(W).astype(dtype))
    m, n = W.shape
    if La is None:
        La = lower_normalized(UA, dtype)
    if Lb is None and UB is not None:
        Lb = lower_normalized(UB, dtype)
    s = np.asarray(s, dtype=np.float64).reshape(-1)
    s_row = np.ascontiguousarray((np.full(m, s[0]) if s.size == 1 else s).astype(dtype))
    s_col = None if alpha is None else np.ascontiguousarray(np.asarray(alpha, dtype=np.float64).astype(dtype))
    if s_col is not None:
        assert s_col.shape == (n,)
    if force is not None:
        force = np.ascontiguousarray(force, dtype=np.int32)
        assert force.shape == (m, n)
    Z = np.zeros((m, n), np.int32)
    V = np.zeros((m, n), dtype)
    Y = np.zeros((m, n), np.float64)
    D = np.zeros((m, n), dtype)
    rc = _load(tag)(m, n, _ptr(W), _ptr(Lb), _ptr(La), _ptr(s_row), _ptr(s_col), 0 if bits is None else int(bits),
                    _ptr(force), _ptr(Z), _ptr(V), _ptr(Y), _ptr(D), int(threads))
    if rc != 0:
        raise MemoryError("o3_solve could not allocate its scratch buffer")
    return (Z if bits is None else Z.astype(np.int8)), V, Y, D
