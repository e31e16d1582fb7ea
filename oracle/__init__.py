"""CPU oracle for C = A * B and C = alpha * op(A) * op(B) + beta * C
(float32 inputs, double accumulation).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the library never does. It is a thin ctypes wrapper
over ``oracle.c`` (plain C, gcc, OpenMP), which shares no code with the GPU
path. The arithmetic and its citations are in ``oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(src: str = _SRC, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-Werror", *extra_flags, src,
           "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_entries.argtypes = [i64, vp, vp, i64, vp, i64, vp, i64, vp, vp]
    lib.oracle_gemm_entries.restype = ctypes.c_int
    d = ctypes.c_double
    lib.oracle_gemm_ex.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, d, vp, i64, vp, i64, d,
                                   vp, i64, vp, i64, vp, i64]
    lib.oracle_gemm_ex.restype = ctypes.c_int
    lib.oracle_gemm_ex_entries.argtypes = [ctypes.c_int, ctypes.c_int, i64, vp, vp, i64, d, vp, i64, vp, i64,
                                           d, vp, i64, vp, vp]
    lib.oracle_gemm_ex_entries.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the compiled oracle, building it first if no library exists."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _rows_view(x: np.ndarray, rows: int, cols: int):
    """(pointer, leading dimension) of a row-major float32 matrix view."""
    if x.dtype != np.float32:
        raise TypeError("oracle inputs must be float32")
    if x.ndim != 2 or x.shape[0] < rows or x.shape[1] < cols:
        raise ValueError("operand smaller than its logical shape")
    if rows == 0 or cols == 0:
        return x.ctypes.data, max(cols, 1)
    # A stride along a dimension of extent 1 is never used (numpy leaves it
    # arbitrary in views such as the transpose of a single row).
    if (cols > 1 and x.strides[1] != 4) or (rows > 1 and (x.strides[0] % 4 or x.strides[0] < 4 * cols)):
        raise ValueError("operand must be row-major with unit column stride")
    return x.ctypes.data, (x.strides[0] // 4 if rows > 1 else max(cols, 1))


def gemm(A: np.ndarray, B: np.ndarray, with_abs: bool = False, lib=None):
    """C = A @ B in double (and S = |A| @ |B| if ``with_abs``).

    A is M x K, B is K x N, row-major float32 (views with a row stride larger
    than the row length are accepted and read through their leading dimension).
    """
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    pa, lda = _rows_view(A, M, K)
    pb, ldb = _rows_view(B, K, N)
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if with_abs else None
    rc = lib.oracle_gemm(M, N, K, pa, max(lda, 1), pb, max(ldb, 1),
                         C.ctypes.data, max(N, 1),
                         S.ctypes.data if with_abs else None, max(N, 1))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm returned {rc}")
    return (C, S) if with_abs else C


def gemm_entries(A: np.ndarray, B: np.ndarray, rows, cols, lib=None):
    """(C[rows[e], cols[e]], S[rows[e], cols[e]]) for each e, in double."""
    lib = lib or load()
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    if rows.size and (rows.min() < 0 or rows.max() >= M
                      or cols.min() < 0 or cols.max() >= N):
        raise IndexError("entry outside the product")
    pa, lda = _rows_view(A, M, K)
    pb, ldb = _rows_view(B, K, N)
    out = np.empty(rows.size, dtype=np.float64)
    sabs = np.empty(rows.size, dtype=np.float64)
    rc = lib.oracle_gemm_entries(rows.size, rows.ctypes.data, cols.ctypes.data,
                                 K, pa, max(lda, 1), pb, max(ldb, 1),
                                 out.ctypes.data, sabs.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_entries returned {rc}")
    return out, sabs


def gemm_ex(transA: bool, transB: bool, alpha: float, A: np.ndarray, B: np.ndarray,
            beta: float, C: np.ndarray | None, lib=None):
    """(alpha * op(A) @ op(B) + beta * C, error scale S) in double.

    A is stored M x K (or K x M when transA), B K x N (or N x K when transB);
    C (M x N float32) is read only when beta != 0.
    """
    lib = lib or load()
    if transA:
        K, M = A.shape
    else:
        M, K = A.shape
    if transB:
        N, K2 = B.shape
    else:
        K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    pa, lda = _rows_view(A, *A.shape)
    pb, ldb = _rows_view(B, *B.shape)
    if beta != 0.0:
        if C is None or C.shape != (M, N):
            raise ValueError("C must be M x N when beta != 0")
        pc, ldc = _rows_view(C, M, N)
    else:
        pc, ldc = None, max(N, 1)
    out = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_gemm_ex(int(bool(transA)), int(bool(transB)), M, N, K, float(alpha),
                            pa, max(lda, 1), pb, max(ldb, 1), float(beta), pc, max(ldc, 1),
                            out.ctypes.data, max(N, 1), S.ctypes.data, max(N, 1))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_ex returned {rc}")
    return out, S


def gemm_ex_entries(transA: bool, transB: bool, alpha: float, A: np.ndarray, B: np.ndarray,
                    beta: float, C: np.ndarray | None, rows, cols, lib=None):
    """Selected elements (rows[e], cols[e]) of gemm_ex's result and their
    error scales, each formed exactly as gemm_ex forms it."""
    lib = lib or load()
    M, K = (A.shape[1], A.shape[0]) if transA else A.shape
    N, K2 = (B.shape[0], B.shape[1]) if transB else (B.shape[1], B.shape[0])
    if K2 != K:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("entry outside the M x N result")
    pa, lda = _rows_view(A, *A.shape)
    pb, ldb = _rows_view(B, *B.shape)
    if beta != 0.0:
        if C is None or C.shape != (M, N):
            raise ValueError("C must be M x N when beta != 0")
        pc, ldc = _rows_view(C, M, N)
    else:
        pc, ldc = None, 1
    out = np.empty(rows.size, dtype=np.float64)
    S = np.empty(rows.size, dtype=np.float64)
    rc = lib.oracle_gemm_ex_entries(int(bool(transA)), int(bool(transB)), rows.size, rows.ctypes.data,
                                    cols.ctypes.data, K, float(alpha), pa, max(lda, 1), pb, max(ldb, 1),
                                    float(beta), pc, max(ldc, 1), out.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_ex_entries returned {rc}")
    return out, S


def lowp_to_float32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of 16-bit encodings: the operands of the
    reduced-precision workload widen to float32 without rounding, after which
    the product is gemm / gemm_ex of the widened matrices.

    bf16: the encoding is the upper half of a float32 encoding.
    f16: IEEE 754 binary16, decoded from its fields: sign s, 5-bit exponent e,
    10-bit fraction f; value (-1)^s * 2^(e-15) * (1 + f/2^10) for 0 < e < 31,
    (-1)^s * 2^-14 * (f/2^10) for e = 0, infinity or NaN for e = 31.
    """
    b = np.asarray(bits).astype(np.uint32)
    if dtype == "bf16":
        return np.ascontiguousarray((b << np.uint32(16)).view(np.float32))
    if dtype == "f16":
        sign = np.where(b >> np.uint32(15), -1.0, 1.0)
        e = ((b >> np.uint32(10)) & np.uint32(0x1F)).astype(np.int64)
        f = (b & np.uint32(0x3FF)).astype(np.float64)
        normal = np.ldexp(1.0 + f / 1024.0, e - 15)
        sub = np.ldexp(f / 1024.0, -14)
        special = np.where(f == 0, np.inf, np.nan)
        v = np.where(e == 0, sub, np.where(e == 31, special, normal))
        return np.ascontiguousarray((sign * v).astype(np.float32))
    raise ValueError(f"unknown 16-bit type {dtype!r}")


def num_threads(lib=None) -> int:
    return (lib or load()).oracle_num_threads()
