"""Python binding of libgemm355: C = alpha*A@B + beta*C on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libgemm355.so`` behind the C ABI of ``include/gemm355.h``; torch
supplies device memory and the current stream.  There is no fallback: if the
library is not built, importing the compute functions raises.

Two levels:
  * ``gemm_f32(A, B, C, alpha, beta)`` / ``gemm_f16r_f32acc(...)`` take torch
    float32 tensors on the GPU (row-major, unit column stride; the leading
    dimension is ``stride(0)``) and enqueue on torch's current stream;
  * ``lib()`` returns the ctypes handle with typed signatures, for raw pointers.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MODE_F32", "MODE_F16R", "Gemm355Error", "lib", "library_path", "gemm", "gemm_f32",
    "gemm_f16r_f32acc", "gemm_noalloc", "tune", "get_config", "set_config", "parse_config", "list_configs",
    "cache_load", "cache_save", "cache_clear", "strerror", "version", "EXPORTS",
]

MODE_F32 = 0
MODE_F16R = 1
_MODES = {"f32": MODE_F32, "f16r": MODE_F16R}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgemm355.so"
_lib = None

_i64, _f32, _p, _cp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_char_p

# name -> (restype, argtypes): every symbol include/gemm355.h declares.
EXPORTS = {
    "gemm_f32": (ctypes.c_int, [_i64, _i64, _i64, _f32, _p, _i64, _p, _i64, _f32, _p, _i64, _p]),
    "gemm_f16r_f32acc": (ctypes.c_int,
                         [_i64, _i64, _i64, _f32, _p, _i64, _p, _i64, _f32, _p, _i64, _p]),
    "gemm_f32_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _f32, _p, _i64,
                                   _p, _i64, _f32, _p, _i64, _p]),
    "gemm_f16r_f32acc_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _f32, _p,
                                           _i64, _p, _i64, _f32, _p, _i64, _p]),
    "gemm_f16r_f16out": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _f32, _p,
                                        _i64, _p, _i64, _f32, _p, _i64, _p]),
    "gemm355_gemm_noalloc": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64,
                                            _i64, _f32, _p, _i64, _p, _i64, _f32, _p, _i64, _p]),
    "gemm355_tune": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _p, _i64, _p, _i64, _f32,
                                    _i64, _p]),
    "gemm355_tune_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64, _i64,
                                       _p, _i64, _p, _i64, _f32, _i64, _p]),
    "gemm355_get_config": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _i64,
                                          _f32, _p, ctypes.c_size_t]),
    "gemm355_get_config_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64,
                                             _i64, _i64, _i64, _i64, _f32, _p, ctypes.c_size_t]),
    "gemm355_get_plan_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64,
                                           _i64, _i64, _i64, _i64, _f32, _p, ctypes.c_size_t]),
    "gemm355_set_config": (ctypes.c_int, [ctypes.c_int, _cp]),
    "gemm355_parse_config": (ctypes.c_int, [ctypes.c_int, _cp, _p, ctypes.c_size_t]),
    "gemm355_list_configs": (ctypes.c_int, [ctypes.c_int, _p, ctypes.c_size_t]),
    "gemm355_cache_load": (ctypes.c_int, [_cp]),
    "gemm355_cache_save": (ctypes.c_int, [_cp]),
    "gemm355_cache_clear": (None, []),
    "gemm355_strerror": (_cp, [ctypes.c_int]),
    "gemm355_version": (_cp, []),
    "gemm355_roof_mfma": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, ctypes.c_int, _p,
                                         ctypes.POINTER(ctypes.c_double), _p]),
    "gemm355_roof_fma": (ctypes.c_int, [_i64, ctypes.c_int, _p, ctypes.POINTER(ctypes.c_double), _p]),
    "gemm355_roof_hbm": (ctypes.c_int, [_p, _i64, ctypes.c_int, _p, _p]),
    "gemm355_copy_f32": (ctypes.c_int, [_p, _p, _i64, _p]),
}


class Gemm355Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: status {status} ({strerror(status)})")


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def lib():
    """The loaded libgemm355 (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "or python gemm_tiled_amd/_build.py")
    handle = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    _lib = handle
    return handle


def strerror(status: int) -> str:
    return lib().gemm355_strerror(int(status)).decode()


def version() -> str:
    return lib().gemm355_version().decode()


def _mode(mode) -> int:
    if isinstance(mode, str):
        return _MODES[mode]
    return int(mode)


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _matrix(t, name, rows=None, cols=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    r, c = t.shape
    if (rows is not None and r != rows) or (cols is not None and c != cols):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected ({rows}, {cols})")
    if c > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    ld = t.stride(0) if r > 1 else max(c, 1)
    return ld


def _operands(A, B, C, transa, transb):
    """Shapes and leading dimensions of one call: A is stored M x K (K x M when
    transa), B K x N (N x K when transb)."""
    if transa:
        K, M = A.shape
    else:
        M, K = A.shape
    N = B.shape[0] if transb else B.shape[1]
    lda = _matrix(A, "A", *((K, M) if transa else (M, K)))
    ldb = _matrix(B, "B", *((N, K) if transb else (K, N)))
    ldc = _matrix(C, "C", M, N)
    return M, N, K, lda, ldb, ldc


def gemm(mode, A, B, C, alpha=1.0, beta=0.0, stream=None, transa=False, transb=False):
    """C = alpha*op(A)@op(B) + beta*C in place, on torch's current stream (or
    `stream`); op(X) = X, or X transposed when transa / transb (A then holds
    K x M, B N x K, both row-major)."""
    M, N, K, lda, ldb, ldc = _operands(A, B, C, transa, transb)
    if (A.numel() and A.device != C.device) or (B.numel() and B.device != C.device):
        raise ValueError("A, B and C must be on the same device")
    ptrs = (float(alpha), A.data_ptr() or None, lda, B.data_ptr() or None, ldb, float(beta),
            C.data_ptr() or None, ldc, _stream_ptr(stream))
    f32 = _mode(mode) == MODE_F32
    if transa or transb:
        name = "gemm_f32_ex" if f32 else "gemm_f16r_f32acc_ex"
        st = getattr(lib(), name)(int(bool(transa)), int(bool(transb)), M, N, K, *ptrs)
    else:
        name = "gemm_f32" if f32 else "gemm_f16r_f32acc"
        st = getattr(lib(), name)(M, N, K, *ptrs)
    if st != 0:
        raise Gemm355Error(st, name)
    return C


def gemm_noalloc(mode, A, B, C, alpha=1.0, beta=0.0, stream=None, transa=False, transb=False):
    """gemm() through gemm355_gemm_noalloc: the same result, with the library's
    scratch taken from its fixed per-GPU array instead of allocated memory
    (calls that overlap on one GPU race; see include/gemm355.h)."""
    M, N, K, lda, ldb, ldc = _operands(A, B, C, transa, transb)
    if (A.numel() and A.device != C.device) or (B.numel() and B.device != C.device):
        raise ValueError("A, B and C must be on the same device")
    st = lib().gemm355_gemm_noalloc(_mode(mode), int(bool(transa)), int(bool(transb)), M, N, K,
                                    float(alpha), A.data_ptr() or None, lda, B.data_ptr() or None,
                                    ldb, float(beta), C.data_ptr() or None, ldc,
                                    _stream_ptr(stream))
    if st != 0:
        raise Gemm355Error(st, "gemm355_gemm_noalloc")
    return C


def gemm_f32(A, B, C, alpha=1.0, beta=0.0, stream=None, transa=False, transb=False):
    return gemm(MODE_F32, A, B, C, alpha, beta, stream, transa, transb)


def gemm_f16r_f32acc(A, B, C, alpha=1.0, beta=0.0, stream=None, transa=False, transb=False):
    return gemm(MODE_F16R, A, B, C, alpha, beta, stream, transa, transb)


def gemm_f16r_f16out(A, B, C16, alpha=1.0, beta=0.0, stream=None, transa=False, transb=False):
    """C16 = alpha*op(A)@op(B) + beta*C16 with A, B float32 (rounded to binary16
    inside) and C16 a float16 tensor (row-major), the result rounded to
    nearest even."""
    import torch
    if not isinstance(C16, torch.Tensor) or C16.dtype != torch.float16 or C16.dim() != 2:
        raise TypeError("C16 must be a 2-D float16 tensor")
    M, N = C16.shape
    if C16.is_cuda is False or (N > 1 and C16.stride(1) != 1):
        raise ValueError("C16 must be a row-major tensor on the GPU")
    ldc = C16.stride(0) if M > 1 else max(N, 1)
    K = A.shape[0] if transa else A.shape[1]
    lda = _matrix(A, "A", *((K, M) if transa else (M, K)))
    ldb = _matrix(B, "B", *((N, K) if transb else (K, N)))
    st = lib().gemm_f16r_f16out(int(bool(transa)), int(bool(transb)), M, N, K, float(alpha),
                                A.data_ptr() or None, lda, B.data_ptr() or None, ldb, float(beta),
                                C16.data_ptr() or None, ldc, _stream_ptr(stream))
    if st != 0:
        raise Gemm355Error(st, "gemm_f16r_f16out")
    return C16


def tune(mode, A, B, C, beta=0.0, stream=None, transa=False, transb=False):
    """Autotune the tile configuration for this call's shape and layout; C is
    not touched."""
    M, N, K, lda, ldb, ldc = _operands(A, B, C, transa, transb)
    st = lib().gemm355_tune_ex(_mode(mode), int(bool(transa)), int(bool(transb)), M, N, K,
                               A.data_ptr() or None, lda, B.data_ptr() or None, ldb, float(beta),
                               ldc, _stream_ptr(stream))
    if st != 0:
        raise Gemm355Error(st, "gemm355_tune_ex")


def get_config(mode, M, N, K, lda=None, ldb=None, ldc=None, beta=0.0, transa=False,
               transb=False) -> str:
    buf = ctypes.create_string_buffer(256)
    lda = lda or max(M if transa else K, 1)
    ldb = ldb or max(K if transb else N, 1)
    st = lib().gemm355_get_config_ex(_mode(mode), int(bool(transa)), int(bool(transb)), M, N, K,
                                     lda, ldb, ldc or max(N, 1), float(beta), buf, 256)
    if st != 0:
        raise Gemm355Error(st, "gemm355_get_config_ex")
    return buf.value.decode()


def get_plan(mode, M, N, K, lda=None, ldb=None, ldc=None, beta=0.0, transa=False,
             transb=False) -> str:
    """How the call would run: "form=... block=MBxNBxKB" (see gemm355_get_plan_ex)."""
    buf = ctypes.create_string_buffer(256)
    lda = lda or max(M if transa else K, 1)
    ldb = ldb or max(K if transb else N, 1)
    st = lib().gemm355_get_plan_ex(_mode(mode), int(bool(transa)), int(bool(transb)), M, N, K,
                                   lda, ldb, ldc or max(N, 1), float(beta), buf, 256)
    if st != 0:
        raise Gemm355Error(st, "gemm355_get_plan_ex")
    return buf.value.decode()


def set_config(mode, spec: str | None):
    st = lib().gemm355_set_config(_mode(mode), spec.encode() if spec else None)
    if st != 0:
        raise Gemm355Error(st, "gemm355_set_config")


def parse_config(mode, spec: str) -> str:
    buf = ctypes.create_string_buffer(256)
    st = lib().gemm355_parse_config(_mode(mode), spec.encode(), buf, 256)
    if st != 0:
        raise Gemm355Error(st, "gemm355_parse_config")
    return buf.value.decode()


def list_configs(mode) -> list[str]:
    buf = ctypes.create_string_buffer(8192)
    n = lib().gemm355_list_configs(_mode(mode), buf, 8192)
    if n < 0:
        raise Gemm355Error(n, "gemm355_list_configs")
    return [s for s in buf.value.decode().split("\n") if s]


def cache_load(path: str) -> int:
    n = lib().gemm355_cache_load(path.encode())
    if n < 0:
        raise Gemm355Error(n, "gemm355_cache_load")
    return n


def cache_save(path: str | None = None) -> int:
    n = lib().gemm355_cache_save(path.encode() if path else None)
    if n < 0:
        raise Gemm355Error(n, "gemm355_cache_save")
    return n


def cache_clear():
    lib().gemm355_cache_clear()
