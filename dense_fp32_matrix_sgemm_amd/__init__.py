"""FP32 matrix multiply C = A * B, and C = alpha * op(A) * op(B) + beta * C,
on AMD MI355X (gfx950).

Python binding of the C ABI declared in ``include/sgemm.h``: argument
marshalling only. Every step of the product runs in the HIP kernels of
``lib/libsgemm.so``; there is no CPU path. PyTorch supplies device buffers
and streams.

Raw entry points (same names and arguments as the C ABI):
    sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream, variant) -> status
    sgemm_check_args(M, N, K, A, lda, B, ldb, C, ldc, variant) -> status
    sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
             stream, variant) -> status
    sgemm_ex_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                        C, ldc, variant) -> status
    sgemm_ex_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                     C, ldc, stream, variant) -> status
                                 (scratch in the library's static buffer)
    sgemm_ex_noalloc_check_args(..., variant, cus) -> status
    sgemm_ex_noalloc_scratch_bytes() -> int
    sgemm_lp(dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
             ldc, stream) -> status      (A, B: bf16 or f16 encodings)
    sgemm_lp_check_args(dtype, transA, transB, M, N, K, alpha, A, lda, B,
                        ldb, beta, C, ldc) -> status
    sgemm_status_string(status) -> str
    sgemm_variant_name(variant) -> str | None
    sgemm_best_variant(M, N, K) -> variant
    sgemm_mfma_tile(M, N, K, cus=0) -> (BM, BN)
    sgemm_mfma_shape(M, N, K, cus=0) -> (BM, BN, BK, waves M, waves N, k sets)
    sgemm_regblock_tile(M, N, cus=0) -> tile edge of the REGBLOCK variant
Pointers are integers (device addresses); ``stream`` is a hipStream_t as an
integer (0 = null stream).

Tensor convenience:
    matmul(A, B, out=None, variant="best") -> C
    gemm(A, B, C=None, alpha=1.0, beta=0.0, variant="best") -> C
      (A, B float32; or both bfloat16 or both float16, summed in float32)
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libsgemm.so")

# Status codes (sgemm_status).
SGEMM_OK = 0
SGEMM_ERR_DIM = -1
SGEMM_ERR_LD = -2
SGEMM_ERR_NULL = -3
SGEMM_ERR_VARIANT = -4
SGEMM_ERR_LAUNCH = -5
SGEMM_ERR_DEVICE = -6
SGEMM_ERR_ALIAS = -7
SGEMM_ERR_OP = -8
SGEMM_ERR_DTYPE = -9
SGEMM_ERR_SCRATCH = -10

# 16-bit operand types (sgemm_lp_type).
SGEMM_LP_BF16 = 1
SGEMM_LP_F16 = 2
LP_TYPES = {"bf16": SGEMM_LP_BF16, "f16": SGEMM_LP_F16}

# Transpose flags (sgemm_op).
SGEMM_OP_N = 0
SGEMM_OP_T = 1

# Variant codes (sgemm_variant).
SGEMM_BEST = -1
SGEMM_NAIVE = 0
SGEMM_TILED = 1
SGEMM_REGBLOCK = 2
SGEMM_MFMA = 3
SGEMM_TILED_T8 = 4
SGEMM_TILED_T16 = 5
SGEMM_TILED_T32 = 6
VARIANTS = {"best": SGEMM_BEST, "naive": SGEMM_NAIVE, "tiled": SGEMM_TILED,
            "regblock": SGEMM_REGBLOCK, "mfma": SGEMM_MFMA,
            "tiled8": SGEMM_TILED_T8, "tiled16": SGEMM_TILED_T16, "tiled32": SGEMM_TILED_T32}

# Symbols the shared library exports (the functions of include/sgemm.h).
EXPORTS = ("sgemm", "sgemm_check_args", "sgemm_ex", "sgemm_ex_check_args", "sgemm_ex_ws", "sgemm_ex_ws_check_args",
           "sgemm_ex_workspace_size", "sgemm_ex_noalloc", "sgemm_ex_noalloc_check_args",
           "sgemm_ex_noalloc_scratch_bytes", "sgemm_lp", "sgemm_lp_check_args", "sgemm_status_string", "sgemm_variant_name",
           "sgemm_best_variant", "sgemm_mfma_tile", "sgemm_mfma_shape", "sgemm_regblock_tile")

_lib = None


class SgemmError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(f"sgemm status {status}: {sgemm_status_string(status)}")


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libsgemm.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    i, vp = ctypes.c_int, ctypes.c_void_p
    lib.sgemm.argtypes = [i, i, i, vp, i, vp, i, vp, i, vp, i]
    lib.sgemm.restype = i
    lib.sgemm_check_args.argtypes = [i, i, i, vp, i, vp, i, vp, i, i]
    lib.sgemm_check_args.restype = i
    f = ctypes.c_float
    lib.sgemm_ex.argtypes = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp, i]
    lib.sgemm_ex.restype = i
    lib.sgemm_ex_check_args.argtypes = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, i]
    lib.sgemm_ex_check_args.restype = i
    sz = ctypes.c_size_t
    lib.sgemm_ex_ws.argtypes = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp, sz, vp, i]
    lib.sgemm_ex_ws.restype = i
    lib.sgemm_ex_ws_check_args.argtypes = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp, sz, i]
    lib.sgemm_ex_ws_check_args.restype = i
    lib.sgemm_ex_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.sgemm_ex_workspace_size.restype = sz
    lib.sgemm_ex_noalloc.argtypes = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp, i]
    lib.sgemm_ex_noalloc.restype = i
    lib.sgemm_ex_noalloc_check_args.argtypes = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, i, i]
    lib.sgemm_ex_noalloc_check_args.restype = i
    lib.sgemm_ex_noalloc_scratch_bytes.argtypes = []
    lib.sgemm_ex_noalloc_scratch_bytes.restype = sz
    lib.sgemm_lp.argtypes = [i, i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp]
    lib.sgemm_lp.restype = i
    lib.sgemm_lp_check_args.argtypes = [i, i, i, i, i, i, f, vp, i, vp, i, f, vp, i]
    lib.sgemm_lp_check_args.restype = i
    lib.sgemm_status_string.argtypes = [i]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_variant_name.argtypes = [i]
    lib.sgemm_variant_name.restype = ctypes.c_char_p
    lib.sgemm_best_variant.argtypes = [i, i, i]
    lib.sgemm_best_variant.restype = i
    ip = ctypes.POINTER(ctypes.c_int)
    lib.sgemm_mfma_tile.argtypes = [i, i, i, i, ip, ip]
    lib.sgemm_mfma_tile.restype = i
    lib.sgemm_mfma_shape.argtypes = [i, i, i, i, ip]
    lib.sgemm_mfma_shape.restype = i
    lib.sgemm_regblock_tile.argtypes = [i, i, i]
    lib.sgemm_regblock_tile.restype = i
    if path is None:
        _lib = lib
    return lib


def sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream, variant) -> int:
    return load_library().sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream, variant)


def sgemm_check_args(M, N, K, A, lda, B, ldb, C, ldc, variant) -> int:
    return load_library().sgemm_check_args(M, N, K, A, lda, B, ldb, C, ldc, variant)


def sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant) -> int:
    return load_library().sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                   stream, variant)


def sgemm_ex_ws(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes, stream,
                variant) -> int:
    return load_library().sgemm_ex_ws(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                      workspace_bytes, stream, variant)


def sgemm_ex_ws_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes,
                           variant) -> int:
    return load_library().sgemm_ex_ws_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                                 workspace, workspace_bytes, variant)


def sgemm_ex_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant) -> int:
    return load_library().sgemm_ex_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                                           variant)


def sgemm_ex_noalloc_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant,
                                cus) -> int:
    return load_library().sgemm_ex_noalloc_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                                      variant, cus)


def sgemm_ex_noalloc_scratch_bytes() -> int:
    """Bytes of the static device buffer sgemm_ex_noalloc works in."""
    return int(load_library().sgemm_ex_noalloc_scratch_bytes())


def sgemm_ex_workspace_size(transA: int, transB: int, M: int, N: int, K: int, cus: int = 0) -> int:
    """Workspace bytes sgemm_ex_ws needs for this product (0: it would not split it)."""
    return int(load_library().sgemm_ex_workspace_size(transA, transB, M, N, K, cus))


def sgemm_ex_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant) -> int:
    return load_library().sgemm_ex_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                                              C, ldc, variant)


def sgemm_lp(dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream) -> int:
    return load_library().sgemm_lp(dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_lp_check_args(dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc) -> int:
    return load_library().sgemm_lp_check_args(dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)


def sgemm_status_string(status: int) -> str:
    return load_library().sgemm_status_string(status).decode()


def sgemm_variant_name(variant: int):
    r = load_library().sgemm_variant_name(variant)
    return None if r is None else r.decode()


def sgemm_best_variant(M: int, N: int, K: int) -> int:
    return load_library().sgemm_best_variant(M, N, K)


def sgemm_mfma_shape(M: int, N: int, K: int, cus: int = 0):
    """(BM, BN, BK, waves along M, waves along N, k sets) of the MFMA kernel for an M x N x K product."""
    shape = (ctypes.c_int * 6)()
    rc = load_library().sgemm_mfma_shape(M, N, K, cus, shape)
    if rc != SGEMM_OK:
        raise SgemmError(rc)
    return tuple(shape)


def sgemm_mfma_tile(M: int, N: int, K: int, cus: int = 0):
    """(BM, BN) of the interior tile the MFMA variant uses for M x N x K."""
    bm, bn = ctypes.c_int(), ctypes.c_int()
    rc = load_library().sgemm_mfma_tile(M, N, K, cus, ctypes.byref(bm), ctypes.byref(bn))
    if rc != SGEMM_OK:
        raise SgemmError(rc)
    return bm.value, bn.value


def sgemm_regblock_tile(M: int, N: int, cus: int = 0) -> int:
    """Edge of the square tile (128, 64 or 32) the REGBLOCK variant uses for M x N."""
    rc = load_library().sgemm_regblock_tile(M, N, cus)
    if rc < 0:
        raise SgemmError(rc)
    return rc


def _variant_code(variant) -> int:
    if isinstance(variant, str):
        if variant not in VARIANTS:
            raise ValueError(f"unknown variant {variant!r}; one of {sorted(VARIANTS)}")
        return VARIANTS[variant]
    return int(variant)


def _storage(t, name):
    """(transpose flag, leading dimension) under which the C ABI reads the
    2-D tensor t as its logical matrix: row-major (unit column stride, rows
    at least a row apart) is read as is; column-major (unit row stride: a
    transposed view of a row-major tensor) is read as the transpose of its
    row-major storage. Row-major is preferred when both apply."""
    rows, cols = t.shape
    s0, s1 = t.stride()
    if rows == 0 or cols == 0:
        return SGEMM_OP_N, max(cols, 1)
    if (cols == 1 or s1 == 1) and (rows == 1 or s0 >= cols):
        return SGEMM_OP_N, s0 if rows > 1 else cols
    if (rows == 1 or s0 == 1) and (cols == 1 or s1 >= rows):
        return SGEMM_OP_T, s1 if cols > 1 else rows
    raise ValueError(f"{name} must be row-major or column-major (strides {(s0, s1)})")


_INT32_MAX = 2**31 - 1


def _check_int32(**sizes):
    """The C ABI takes sizes and leading dimensions as C int; ctypes would
    wrap a larger value silently (2**32 + 8 arrives as 8), so refuse it."""
    for name, v in sizes.items():
        if not 0 <= v <= _INT32_MAX:
            raise ValueError(f"{name} = {v} is outside the C ABI's int range [0, {_INT32_MAX}]")


def _check_tensor(t, name):
    import torch

    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")


def gemm(A, B, C=None, alpha=1.0, beta=0.0, variant="best", workspace=None):
    """C = alpha * A @ B + beta * C for float32 GPU tensors A (M x K), B (K x N).

    A and B may be row-major or column-major views (a transposed view such
    as ``X.t()`` is passed to the kernels as a transposed operand, without a
    copy). C (M x N, row-major, rows possibly padded) is updated in place; it
    is read only when beta != 0, and allocated when None (then beta must be
    0). The kernels are enqueued on the current stream of A's device.
    ``workspace``, a contiguous GPU tensor on A's device, lets the library use
    the split schedule (sgemm_ex_ws) where it is faster; its size in bytes
    should be at least sgemm_ex_workspace_size() for the product.
    """
    import torch

    lp = {torch.bfloat16: SGEMM_LP_BF16, torch.float16: SGEMM_LP_F16}
    if isinstance(A, torch.Tensor) and A.dtype in lp:
        return _gemm_lp(A, B, C, alpha, beta, lp[A.dtype])
    _check_tensor(A, "A")
    _check_tensor(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} @ {tuple(B.shape)}")
    if B.device != A.device:
        raise ValueError("A and B are on different devices")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    else:
        _check_tensor(C, "C")
        if C.device != A.device or tuple(C.shape) != (M, N):
            raise ValueError("C must be an M x N tensor on A's device")
    ta, lda = _storage(A, "A")
    tb, ldb = _storage(B, "B")
    tc, ldc = _storage(C, "C")
    if tc != SGEMM_OP_N:
        raise ValueError("C must be row-major (unit column stride)")
    _check_int32(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    with torch.cuda.device(A.device):
        stream = torch.cuda.current_stream(A.device).cuda_stream
        if workspace is None:
            rc = sgemm_ex(ta, tb, M, N, K, float(alpha), A.data_ptr() or None, lda,
                          B.data_ptr() or None, ldb, float(beta), C.data_ptr() or None, ldc,
                          stream or None, _variant_code(variant))
        else:
            if not isinstance(workspace, torch.Tensor) or workspace.device != A.device or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous tensor on A's device")
            rc = sgemm_ex_ws(ta, tb, M, N, K, float(alpha), A.data_ptr() or None, lda,
                             B.data_ptr() or None, ldb, float(beta), C.data_ptr() or None, ldc,
                             workspace.data_ptr() or None, workspace.numel() * workspace.element_size(),
                             stream or None, _variant_code(variant))
    if rc != SGEMM_OK:
        raise SgemmError(rc)
    return C


def _gemm_lp(A, B, C, alpha, beta, dtype):
    """gemm() for bfloat16 / float16 operands: FP32 result and accumulation."""
    import torch

    for name, t in (("A", A), ("B", B)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise TypeError(f"{name} must be a 2-D torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device")
    if B.dtype != A.dtype:
        raise TypeError(f"A and B must have one 16-bit type, got {A.dtype} and {B.dtype}")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} @ {tuple(B.shape)}")
    if B.device != A.device:
        raise ValueError("A and B are on different devices")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    else:
        _check_tensor(C, "C")
        if C.device != A.device or tuple(C.shape) != (M, N):
            raise ValueError("C must be an M x N float32 tensor on A's device")
    ta, lda = _storage(A, "A")
    tb, ldb = _storage(B, "B")
    tc, ldc = _storage(C, "C")
    if tc != SGEMM_OP_N:
        raise ValueError("C must be row-major (unit column stride)")
    _check_int32(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    with torch.cuda.device(A.device):
        stream = torch.cuda.current_stream(A.device).cuda_stream
        rc = sgemm_lp(dtype, ta, tb, M, N, K, float(alpha), A.data_ptr() or None, lda,
                      B.data_ptr() or None, ldb, float(beta), C.data_ptr() or None, ldc, stream or None)
    if rc != SGEMM_OK:
        raise SgemmError(rc)
    return C


def matmul(A, B, out=None, variant="best"):
    """C = A @ B for float32 GPU tensors A (M x K) and B (K x N).

    Operands may be row-major views with a row stride larger than the row
    length (sub-matrices) or transposed (column-major) views; ``out`` (M x N,
    row-major) is overwritten. The kernel is enqueued on the current stream
    of A's device.
    """
    return gemm(A, B, out, 1.0, 0.0, variant)
