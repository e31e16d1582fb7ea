"""Helpers for the GPU tests: place host matrices in device buffers (optionally
with a larger leading dimension and a misaligning start offset), call the C ABI
through the binding, and read the result back."""

from __future__ import annotations

import numpy as np
import torch

import dense_fp32_matrix_sgemm_amd as sg

SENTINEL = -12345.0


def device_matrix(x: np.ndarray, ld: int | None = None, offset: int = 0,
                  fill: float = float("nan")):
    """A rows x cols device view of ``x`` with leading dimension ``ld`` that
    starts ``offset`` floats into a buffer whose other elements hold ``fill``.
    Returns (view, backing buffer)."""
    rows, cols = x.shape
    ld = max(cols, 1) if ld is None else ld
    buf = torch.full((offset + rows * ld + 8,), fill, dtype=torch.float32)
    view = torch.as_strided(buf, (rows, cols), (ld, 1), offset)
    view.copy_(torch.from_numpy(np.ascontiguousarray(x)))
    dbuf = buf.cuda()
    return torch.as_strided(dbuf, (rows, cols), (ld, 1), offset), dbuf


def gemm(A: np.ndarray, B: np.ndarray, variant, ld_pad=(0, 0, 0), offset=(0, 0, 0),
         stream=None, return_buffer=False):
    """Run the library on copies of A and B; returns C (numpy float32).

    C's buffer starts filled with SENTINEL; with ``return_buffer`` the whole
    backing buffer of C and its (ld, offset) are returned too, so a test can
    check that nothing outside the M x N window was written.
    """
    M, K = A.shape
    N = B.shape[1]
    dA, _ = device_matrix(A, K + ld_pad[0], offset[0])
    dB, _ = device_matrix(B, N + ld_pad[1], offset[1])
    ldc = N + ld_pad[2]
    dC, cbuf = device_matrix(np.full((M, N), SENTINEL, np.float32), ldc, offset[2],
                             fill=SENTINEL)
    s = stream or torch.cuda.current_stream()
    rc = sg.sgemm(M, N, K, dA.data_ptr(), max(K + ld_pad[0], 1), dB.data_ptr(),
                  max(N + ld_pad[1], 1), dC.data_ptr(), max(ldc, 1), s.cuda_stream,
                  sg.VARIANTS[variant] if isinstance(variant, str) else variant)
    if rc != sg.SGEMM_OK:
        raise sg.SgemmError(rc)
    s.synchronize()
    C = dC.cpu().numpy()
    if return_buffer:
        return C, cbuf.cpu().numpy(), max(ldc, 1), offset[2]
    return C


def gemm_ex(transA: bool, transB: bool, alpha: float, A: np.ndarray, B: np.ndarray, beta: float,
            C0: np.ndarray, variant, ld_pad=(0, 0, 0), offset=(0, 0, 0), stream=None,
            return_buffer=False, fill=float("nan"), workspace=None):
    """Run sgemm_ex on copies of the stored operands A, B and the initial C0
    (M x N); returns the updated C (numpy float32).

    A is stored M x K (K x M when transA), B K x N (N x K when transB). The
    padding of every buffer holds ``fill`` (NaN: it must never be read), and
    with ``return_buffer`` the whole backing buffer of C and its (ld, offset)
    come back too. With ``workspace`` (a device tensor) the call is
    sgemm_ex_ws with that workspace.
    """
    M, N = C0.shape
    K = A.shape[0] if transA else A.shape[1]
    lda, ldb, ldc = A.shape[1] + ld_pad[0], B.shape[1] + ld_pad[1], N + ld_pad[2]
    dA, _ = device_matrix(A, lda, offset[0], fill)
    dB, _ = device_matrix(B, ldb, offset[1], fill)
    dC, cbuf = device_matrix(C0, ldc, offset[2], fill=SENTINEL)
    s = stream or torch.cuda.current_stream()
    ta, tb = sg.SGEMM_OP_T if transA else sg.SGEMM_OP_N, sg.SGEMM_OP_T if transB else sg.SGEMM_OP_N
    v = sg.VARIANTS[variant] if isinstance(variant, str) else variant
    if workspace is None:
        rc = sg.sgemm_ex(ta, tb, M, N, K, alpha, dA.data_ptr(), max(lda, 1), dB.data_ptr(), max(ldb, 1), beta,
                         dC.data_ptr(), max(ldc, 1), s.cuda_stream, v)
    else:
        rc = sg.sgemm_ex_ws(ta, tb, M, N, K, alpha, dA.data_ptr(), max(lda, 1), dB.data_ptr(), max(ldb, 1), beta,
                            dC.data_ptr(), max(ldc, 1), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), s.cuda_stream, v)
    if rc != sg.SGEMM_OK:
        raise sg.SgemmError(rc)
    s.synchronize()
    C = dC.cpu().numpy()
    if return_buffer:
        return C, cbuf.cpu().numpy(), max(ldc, 1), offset[2]
    return C


LP_NAN = 0x7FFF  # a NaN encoding in both bf16 and f16


def device_u16(bits: np.ndarray, ld: int | None = None, offset: int = 0, fill: int = LP_NAN):
    """A rows x cols device view of 16-bit encodings ``bits`` (uint16) with
    leading dimension ``ld``, starting ``offset`` elements into a buffer whose
    other elements hold ``fill``. Returns (view, backing buffer)."""
    rows, cols = bits.shape
    ld = max(cols, 1) if ld is None else ld
    buf = torch.full((offset + rows * ld + 8,), np.int16(np.uint16(fill).view(np.int16)).item(), dtype=torch.int16)
    view = torch.as_strided(buf, (rows, cols), (ld, 1), offset)
    view.copy_(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)))
    dbuf = buf.cuda()
    return torch.as_strided(dbuf, (rows, cols), (ld, 1), offset), dbuf


def gemm_lp(dtype: str, transA: bool, transB: bool, alpha: float, A_bits: np.ndarray, B_bits: np.ndarray,
            beta: float, C0: np.ndarray, ld_pad=(0, 0, 0), offset=(0, 0, 0), return_buffer=False):
    """Run sgemm_lp on 16-bit encodings A_bits (stored M x K, or K x M when
    transA) and B_bits (K x N, or N x K when transB) with the float32 C0;
    returns the updated C (numpy float32)."""
    M, N = C0.shape
    K = A_bits.shape[0] if transA else A_bits.shape[1]
    lda, ldb, ldc = A_bits.shape[1] + ld_pad[0], B_bits.shape[1] + ld_pad[1], N + ld_pad[2]
    dA, _ = device_u16(A_bits, lda, offset[0])
    dB, _ = device_u16(B_bits, ldb, offset[1])
    dC, cbuf = device_matrix(C0, ldc, offset[2], fill=SENTINEL)
    s = torch.cuda.current_stream()
    rc = sg.sgemm_lp(sg.LP_TYPES[dtype], sg.SGEMM_OP_T if transA else sg.SGEMM_OP_N,
                     sg.SGEMM_OP_T if transB else sg.SGEMM_OP_N, M, N, K, alpha, dA.data_ptr(), max(lda, 1),
                     dB.data_ptr(), max(ldb, 1), beta, dC.data_ptr(), max(ldc, 1), s.cuda_stream)
    if rc != sg.SGEMM_OK:
        raise sg.SgemmError(rc)
    s.synchronize()
    C = dC.cpu().numpy()
    if return_buffer:
        return C, cbuf.cpu().numpy(), max(ldc, 1), offset[2]
    return C
