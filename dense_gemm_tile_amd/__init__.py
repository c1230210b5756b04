"""Python binding of the MI355X dense GEMM library (C ABI in include/dense_gemm_tile.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libdense_gemm_tile_amd.so. Importing this package loads that
library and fails loudly if it has not been built (there is no CPU fallback).

Pointer arguments accept an int (a device address), None (NULL) or any object
with ``data_ptr()`` (a torch tensor). ``stream`` accepts an int (a hipStream_t
value), None (the default stream) or an object with a ``cuda_stream``
attribute (a torch stream).
"""
from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libdense_gemm_tile_amd.so"
LIB_PATH = os.path.join(_PKG_DIR, LIB_NAME)

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = 1
GEMM_ERR_UNSUPPORTED = 2
GEMM_ERR_ALIAS = 3
GEMM_ERR_HIP = 4
GEMM_DTYPE_F16 = 0
GEMM_DTYPE_BF16 = 1
GEMM_DTYPE_F32_F16 = 2   # float32 A and B, rounded to f16 while staged
GEMM_DTYPE_F32_BF16 = 3  # float32 A and B, rounded to bf16 while staged
GEMM_DTYPE_F8_E4M3 = 4   # 8-bit float codes, OCP E4M3
GEMM_DTYPE_F8_E5M2 = 5   # 8-bit float codes, OCP E5M2

# Every symbol the header declares, with its ctypes signature.
_i64, _int, _f32, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
_SIGNATURES = {
    "gemm": (_int, [_i64, _i64, _i64, _int, _int, _int, _f32, _f32,
                    _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "gemm_validate": (_int, [_i64, _i64, _i64, _int, _int, _int, _f32, _f32,
                             _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64]),
    "gemm_i8": (_int, [_i64, _i64, _i64, _int, _int, ctypes.c_int32, ctypes.c_int32,
                       _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "gemm_i8_validate": (_int, [_i64, _i64, _i64, _int, _int, ctypes.c_int32, ctypes.c_int32,
                                _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64]),
    "gemm_last_error": (ctypes.c_char_p, []),
    "gemm_last_path": (ctypes.c_char_p, []),
    "gemm_tile_order": (_int, [_i64, _i64, _int, ctypes.POINTER(ctypes.c_int32),
                               ctypes.POINTER(ctypes.c_int32)]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built. Build it with `python dense_gemm_tile_amd/build.py` "
            "(hipcc, gfx950); this package has no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


class GemmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"gemm failed with status {code}: {message}")
        self.code = code


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


_DTYPE_CODES = {"f16": GEMM_DTYPE_F16, "bf16": GEMM_DTYPE_BF16, "f32_f16": GEMM_DTYPE_F32_F16,
                "f32_bf16": GEMM_DTYPE_F32_BF16, "f8e4m3": GEMM_DTYPE_F8_E4M3,
                "f8e5m2": GEMM_DTYPE_F8_E5M2}


def _dtype(d):
    if isinstance(d, str):
        return _DTYPE_CODES[d]
    return int(d)


def gemm(M, N, K, dtype, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd,
         stream=None):
    """Enqueue D = alpha*op(A)@op(B) + beta*C; raises GemmError on a non-zero status."""
    st = _lib.gemm(M, N, K, _dtype(dtype), int(transA), int(transB), alpha, beta,
                   _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(D), ldd, _stream(stream))
    if st != GEMM_OK:
        raise GemmError(st, gemm_last_error())


def gemm_status(M, N, K, dtype, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd,
                stream=None) -> int:
    """Same as gemm() but returns the status code instead of raising."""
    return _lib.gemm(M, N, K, _dtype(dtype), int(transA), int(transB), alpha, beta,
                     _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(D), ldd, _stream(stream))


def gemm_validate(M, N, K, dtype, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D,
                  ldd) -> int:
    """Host-only checks and path selection; returns the status code."""
    return _lib.gemm_validate(M, N, K, _dtype(dtype), int(transA), int(transB), alpha, beta,
                              _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(D), ldd)


def gemm_i8(M, N, K, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D, ldd, stream=None):
    """Enqueue the int8 form D = alpha*op(A)@op(B) + beta*C (int32 C/D, integer
    alpha/beta, int32 wraparound); raises GemmError on a non-zero status."""
    st = _lib.gemm_i8(M, N, K, int(transA), int(transB), int(alpha), int(beta), _ptr(A), lda,
                      _ptr(B), ldb, _ptr(C), ldc, _ptr(D), ldd, _stream(stream))
    if st != GEMM_OK:
        raise GemmError(st, gemm_last_error())


def gemm_i8_validate(M, N, K, transA, transB, alpha, beta, A, lda, B, ldb, C, ldc, D,
                     ldd) -> int:
    """Host-only checks of the int8 form; returns the status code."""
    return _lib.gemm_i8_validate(M, N, K, int(transA), int(transB), int(alpha), int(beta),
                                 _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, _ptr(D), ldd)


def gemm_last_error() -> str:
    return _lib.gemm_last_error().decode()


def gemm_last_path() -> str:
    return _lib.gemm_last_path().decode()


def gemm_tile_order(tiles_m: int, tiles_n: int, group_m: int):
    """The scheduler's workgroup -> (tile row, tile column) map, as two lists."""
    n = tiles_m * tiles_n
    tm = (ctypes.c_int32 * max(n, 1))()
    tn = (ctypes.c_int32 * max(n, 1))()
    st = _lib.gemm_tile_order(tiles_m, tiles_n, group_m, tm, tn)
    if st != GEMM_OK:
        raise GemmError(st, gemm_last_error())
    return list(tm[:n]), list(tn[:n])


__all__ = ["gemm_i8", "gemm_i8_validate", "gemm", "gemm_status", "gemm_validate", "gemm_last_error", "gemm_last_path",
           "gemm_tile_order", "GemmError", "GEMM_OK", "GEMM_ERR_INVALID_ARG",
           "GEMM_ERR_UNSUPPORTED", "GEMM_ERR_ALIAS", "GEMM_ERR_HIP", "GEMM_DTYPE_F16",
           "GEMM_DTYPE_BF16", "GEMM_DTYPE_F32_F16", "GEMM_DTYPE_F32_BF16", "GEMM_DTYPE_F8_E4M3",
           "GEMM_DTYPE_F8_E5M2", "LIB_PATH"]
