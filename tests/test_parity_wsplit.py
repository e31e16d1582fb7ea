"""The tiles whose K range is split over their four waves (GPU tests).

Each wave of the work-group holds the whole 64x64, 96x96 or 128x128 tile and
multiplies every fourth chunk of k, reading its operands with buffer loads
whose offsets the kernel forms in 31 bits; the four partial tiles are added
in a fixed order at the end (in two rounds of block rows for the 128x128
tile). Beyond the slab-boundary and edge tests, which run them with every K
around their chunks and at odd widths, these check:
- long K (many chunks per wave, a partial last one) against the oracle;
- that two runs give the same bits (the partial tiles meet in a fixed order);
- operands whose offsets do not fit 31 bits: an operand stored with its free
  index contiguous (B as given, A transposed) spans K rows of its leading
  dimension, so K * ld * 4 bytes past 2^31 sends the product to the
  LDS-staged tile of the same size (the two-set 64x64 tile, the eight-wave
  128x128 tile), which must give the same integer product bit for bit. (The
  bound for an operand stored with k contiguous covers one tile's rows, which
  would need a 16 GiB operand or more to cross.)
"""

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import oracle
import synth
from oracle.check import assert_within
from tests.gpu_util import gemm_ex

pytestmark = pytest.mark.gpu

WSPLIT = (64, 64, 32, 1, 1, 4)
WSPLIT96 = (96, 96, 32, 1, 1, 4)
WSPLIT128 = (128, 128, 16, 1, 1, 4)
# (M, N) with at most one tile of each size per compute unit: 240 of them.
SIZES = [((1024, 960), WSPLIT), ((1536, 1440), WSPLIT96), ((2048, 1920), WSPLIT128)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _stored(x, trans):
    return np.ascontiguousarray(x.T) if trans else x


@pytest.mark.parametrize("pair", [(False, False), (False, True), (True, False), (True, True)],
                         ids=["nn", "nt", "tn", "tt"])
@pytest.mark.parametrize("K", [4096, 4099, 4127])
@pytest.mark.parametrize("mn,shape", SIZES, ids=["64", "96", "128"])
def test_long_k(mn, shape, K, pair):
    M, N = mn
    tA, tB = pair
    assert sg.sgemm_mfma_shape(M, N, K) == shape
    print(f"[wsplit] long K {M}x{N}x{K} pair {pair}", flush=True)
    opA = synth.uniform_pm1(K + 1, (M, K))
    opB = synth.uniform_pm1(K + 2, (K, N))
    C0 = synth.uniform_pm1(K + 3, (M, N))
    A, B = _stored(opA, tA), _stored(opB, tB)
    C = gemm_ex(tA, tB, 1.5, A, B, -0.25, C0, "mfma")
    rng = np.random.default_rng(K)
    rows = np.concatenate([rng.integers(0, M, 1500), np.full(64, M - 1), np.arange(64)])
    cols = np.concatenate([rng.integers(0, N, 1500), np.arange(N - 64, N), np.full(64, N - 1)])
    want, S = oracle.gemm_ex_entries(tA, tB, 1.5, A, B, -0.25, C0, rows, cols)
    assert_within(C[rows, cols], want, S, f"{M}x{N}x{K} {pair}")


@pytest.mark.parametrize("M,shape", [(1024, WSPLIT), (1536, WSPLIT96), (2048, WSPLIT128)], ids=["64", "96", "128"])
def test_repeat_is_bitwise(M, shape):
    N = K = M
    assert sg.sgemm_mfma_shape(M, N, K) == shape
    print(f"[wsplit] repeat {M}^3", flush=True)
    A = torch.from_numpy(synth.uniform01(42, (M, K))).cuda()
    B = torch.from_numpy(synth.uniform01(43, (K, N))).cuda()
    C1 = sg.matmul(A, B, variant="mfma")
    C2 = sg.matmul(A, B, variant="mfma")
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))


def _big_ld_product(M, N, K, trans_a):
    """Small-integer product whose free-index-contiguous operand (B, or A
    transposed) is stored with a leading dimension that puts K * ld * 4 bytes
    just past 2^31."""
    ld = (2 ** 31) // (4 * K) + 64
    assert K * ld * 4 >= 2 ** 31
    Ai = synth.small_int(7, (M, K))
    Bi = synth.small_int(8, (K, N))
    exact = Ai.astype(np.float64) @ Bi.astype(np.float64)  # exact: |sums| < 2^53
    dev = torch.device("cuda")
    big = torch.zeros(K * ld, dtype=torch.float32, device=dev)
    if trans_a:
        dA = torch.as_strided(big, (K, M), (ld, 1))  # A stored K x M
        dA.copy_(torch.from_numpy(np.ascontiguousarray(Ai.T)))
        dB = torch.from_numpy(Bi).to(dev)
        lda, ldb = ld, N
        ta, tb = sg.SGEMM_OP_T, sg.SGEMM_OP_N
    else:
        dA = torch.from_numpy(Ai).to(dev)
        dB = torch.as_strided(big, (K, N), (ld, 1))
        dB.copy_(torch.from_numpy(Bi))
        lda, ldb = K, ld
        ta, tb = sg.SGEMM_OP_N, sg.SGEMM_OP_N
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()
    rc = sg.sgemm_ex(ta, tb, M, N, K, 1.0, dA.data_ptr(), lda, dB.data_ptr(), ldb, 0.0, C.data_ptr(), N,
                     s.cuda_stream, sg.SGEMM_MFMA)
    assert rc == sg.SGEMM_OK, rc
    s.synchronize()
    out = C.cpu().numpy()
    del big, dA, dB, C
    torch.cuda.empty_cache()
    return out, exact


@pytest.mark.parametrize("mnk,shape", [((1000, 1000, 1000), WSPLIT), ((2048, 2048, 64), WSPLIT128)],
                         ids=["64", "128"])
@pytest.mark.parametrize("trans_a", [False, True], ids=["B-as-given", "A-transposed"])
def test_offsets_past_31_bits(mnk, shape, trans_a):
    M, N, K = mnk
    assert sg.sgemm_mfma_shape(M, N, K) == shape
    print(f"[wsplit] 31-bit offsets {M}x{N}x{K}, A transposed {trans_a}", flush=True)
    out, exact = _big_ld_product(M, N, K, trans_a)
    assert np.array_equal(out.astype(np.float64), exact)
