"""Oracle for the persistent GEMM: C = A.B accumulated in fp64 over the
decoded (dequantised) inputs, with the elementwise bound Abs = |A|.|B|.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The product the persistent kernels compute, tile by tile, in "Work Stealing
Scheduler Kernel" (tritonBLAS PR #65; the matmul wrapper passes A, B, C and
the quantised path's a_scale / b_scale) and in "[Feature] Introduce tile
scheduler" (TileLang PR #2441; block-scaled MXFP8, scale shape (1, 1, 128)).
The scheduler changes which workgroup computes a tile, never the value.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build
from .codecs import bf16_to_f64, dequant_fp8_a, dequant_fp8_b

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_gemm_f64.argtypes = [dp, dp, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, dp, dp]
        lib.oracle_gemm_f64.restype = None
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def gemm_f64(A: np.ndarray, B: np.ndarray):
    """(C, Abs) for fp64 A[M][K], B[K][N] via the C oracle (k ascending per element)."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    _load().oracle_gemm_f64(A.ctypes.data_as(dp), B.ctypes.data_as(dp), M, N, K,
                            C.ctypes.data_as(dp), S.ctypes.data_as(dp))
    return C, S


def gemm_f64_sampled(A: np.ndarray, B: np.ndarray, rows, cols):
    """(C, Abs) restricted to rows x cols: the same definition on A[rows], B[:, cols]."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    return gemm_f64(A[rows, :], B[:, cols])


def gemm_naive(A, B):
    """Pure-Python triple loop in fp64 (tiny sizes only); independent of the C oracle."""
    M, K = len(A), len(A[0]) if len(A) else 0
    N = len(B[0]) if len(B) else 0
    C = [[0.0] * N for _ in range(M)]
    S = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = 0.0
            acc_abs = 0.0
            for k in range(K):
                a = float(A[i][k])
                b = float(B[k][j])
                acc += a * b
                acc_abs += abs(a) * abs(b)
            C[i][j] = acc
            S[i][j] = acc_abs
    return C, S


def decode_bf16_operands(a_bits, b_bits):
    return bf16_to_f64(a_bits), bf16_to_f64(b_bits)


def decode_fp8_operands(qa, sa, qb, sb):
    return dequant_fp8_a(qa, sa), dequant_fp8_b(qb, sb)


def gemm_bf16(a_bits, b_bits):
    A, B = decode_bf16_operands(a_bits, b_bits)
    return gemm_f64(A, B)


def gemm_fp8_b128(qa, sa, qb, sb):
    A, B = decode_fp8_operands(qa, sa, qb, sb)
    return gemm_f64(A, B)
