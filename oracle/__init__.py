"""CPU reference (oracle) for C = alpha*A@B + beta*C, f32 and f16r modes.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library never
calls it and shares no code with it.

The arithmetic lives in ``gemm_oracle.c`` (plain C, float64, OpenMP over rows):
a triple loop in i-k-j order, k ascending for every element.  This module only
loads the compiled library and marshals numpy arrays.

What it computes follows the phobos docs page "gemm, f32" (opening paragraph:
C = alpha*A@B + beta*C on f32 matrices; section "The epilogue": alpha*acc +
beta*c_old stored over the same tile) and the page "gemm on tensor cores"
(section "What changes": the operands are rounded to f16, products are summed
in f32).  The reference is kept in float64; the parity bound compares a result
to it elementwise, relative to W = |alpha|*(|r(A)||r(B)|)_ij + |beta||C_ij|.

Pins (tests/test_oracle.py): exact rational brute force on tiny shapes, numpy
float64 matmul at moderate sizes, alpha=0, identity, all-ones A, small integers,
and the f16 rounding exhaustively against the CPU's own float16 conversion.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

MODE_F32 = 0
MODE_F16R = 1
MODES = {"f32": MODE_F32, "f16r": MODE_F16R}

# Parity tolerance of each mode: |C_gpu - C_ref| <= tol * W elementwise.
TOL = {"f32": 1e-5, "f16r": 4e-5}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_f64 = ctypes.c_double
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_rn_f16_bits.argtypes = [_f32]
    lib.oracle_rn_f16_bits.restype = ctypes.c_uint16
    lib.oracle_f16_bits_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_bits_to_double.restype = _f64
    lib.oracle_rn_f16_array.argtypes = [_p, _p, _i64]
    lib.oracle_rn_f16_array.restype = None
    lib.oracle_gemm.argtypes = [ctypes.c_int, _i64, _i64, _i64, _f32, _p, _i64, _p, _i64,
                                _f32, _p, _i64, _p, _p]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_entries.argtypes = [ctypes.c_int, _i64, _f32, _p, _i64, _p, _i64,
                                        _f32, _p, _i64, _p, _p, _i64, _p, _p]
    lib.oracle_gemm_entries.restype = None
    lib.oracle_check.argtypes = [ctypes.c_int, _i64, _i64, _i64, _f32, _p, _i64, _p, _i64,
                                 _f32, _p, _i64, _p, _i64, _f64, _i64, _i64, _p]
    lib.oracle_check.restype = ctypes.c_int
    _lib = lib
    return lib


def _mode(mode):
    return MODES[mode] if isinstance(mode, str) else int(mode)


def _mat(x, name):
    """A row-major float32 matrix view and its leading dimension (elements)."""
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size == 0:
        return x, max(x.shape[1], 1)
    if (x.shape[1] > 1 and x.strides[1] != 4) or x.strides[0] % 4:
        raise ValueError(f"{name} must be row-major with unit column stride")
    ld = max(x.strides[0] // 4, x.shape[1], 1) if x.shape[0] > 1 else max(x.shape[1], 1)
    return x, ld


def _ptr(x):
    return ctypes.c_void_p(x.ctypes.data) if x is not None and x.size else ctypes.c_void_p(0)


def rn_f16_bits(x):
    """IEEE binary16 bits of float32 x, round to nearest, ties to even."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_rn_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_float64(h):
    lib = _load()
    h = np.asarray(h, dtype=np.uint16)
    return np.array([lib.oracle_f16_bits_to_double(int(v)) for v in h.ravel()],
                    dtype=np.float64).reshape(h.shape)


def gemm(mode, A, B, C, alpha, beta):
    """Full reference: (Cref, W) as float64 M x N arrays.  C is not modified."""
    A, lda = _mat(A, "A")
    B, ldb = _mat(B, "B")
    C, ldc = _mat(C, "C")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or C.shape != (M, N):
        raise ValueError("shape mismatch")
    Cref = np.zeros((M, N), dtype=np.float64)
    W = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_gemm(_mode(mode), M, N, K, alpha, _ptr(A), lda, _ptr(B), ldb,
                             beta, _ptr(C), ldc, _ptr(Cref), _ptr(W))
    if rc != 0:
        raise MemoryError("oracle_gemm failed")
    return Cref, W


def entries(mode, A, B, C, alpha, beta, rows, cols):
    """Reference and W for the sampled elements (rows[s], cols[s])."""
    A, lda = _mat(A, "A")
    B, ldb = _mat(B, "B")
    C, ldc = _mat(C, "C")
    K = A.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in shape")
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0] or cols.min() < 0
                      or cols.max() >= B.shape[1]):
        raise IndexError("sample index out of range")
    ref = np.zeros(rows.shape, dtype=np.float64)
    W = np.zeros(rows.shape, dtype=np.float64)
    _load().oracle_gemm_entries(_mode(mode), K, alpha, _ptr(A), lda, _ptr(B), ldb, beta,
                                _ptr(C), ldc, _ptr(rows), _ptr(cols), rows.size,
                                _ptr(ref), _ptr(W))
    return ref, W


def check(mode, A, B, C0, alpha, beta, Cgot, tol=None, rows=None):
    """Compare Cgot with the reference over all rows (or a band rows=(lo, hi)).

    Returns a dict: max_ratio (max |err|/W), n_fail (elements outside tol*W),
    err_max_norm (max|err| / max|ref|) and err_fro (||err|| / ||ref||), the
    lab's two error summaries.
    """
    A, lda = _mat(A, "A")
    B, ldb = _mat(B, "B")
    C0, ldc = _mat(C0, "C0")
    Cgot, ldg = _mat(Cgot, "Cgot")
    M, K = A.shape
    N = B.shape[1]
    if Cgot.shape != (M, N) or C0.shape != (M, N) or B.shape[0] != K:
        raise ValueError("shape mismatch")
    if tol is None:
        tol = TOL[mode] if isinstance(mode, str) else TOL[["f32", "f16r"][mode]]
    lo, hi = (0, M) if rows is None else rows
    stats = np.zeros(6, dtype=np.float64)
    rc = _load().oracle_check(_mode(mode), M, N, K, alpha, _ptr(A), lda, _ptr(B), ldb,
                              beta, _ptr(C0), ldc, _ptr(Cgot), ldg, tol, lo, hi,
                              _ptr(stats))
    if rc != 0:
        raise MemoryError("oracle_check failed")
    max_ratio, n_fail, max_err, max_ref, se, sr = stats
    return {
        "max_ratio": float(max_ratio),
        "n_fail": int(n_fail),
        "tol": float(tol),
        "err_max_norm": float(max_err / max_ref) if max_ref > 0 else float(max_err),
        "err_fro": float(np.sqrt(se / sr)) if sr > 0 else float(np.sqrt(se)),
    }
