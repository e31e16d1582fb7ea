"""Edge tiles of the matrix-core path (GPU tests).

Tiles that cross the bottom or right edge of C run the same loop as the
others, with their reads clamped into the operands and the partial chunk of
a row-contiguous operand read from a shifted address and rotated into place.
These tests run ragged products whose chosen tile shape (each of 256x256,
192x128, 128x192, both 128x128 tiles, 64x64, the 64x64 and 32x32 tiles
whose slabs two wave sets share, and the 64x64, 96x96 and 128x128 tiles whose
K range is split over their four waves) leaves
partial tiles on both edges, for every transpose pair, with alpha and beta,
and the narrowest widths the clamped reads allow (4 to 7) next to the general
path below them. Every comparison is with the
oracle; sampled outputs always include the last rows and columns.
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

PAIRS = [(False, False), (False, True), (True, False), (True, True)]
PAIR_IDS = ["nn", "nt", "tn", "tt"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _stored(x, trans):
    return np.ascontiguousarray(x.T) if trans else x


# (M, N, K) and the kernel shape the library picks for it (BM, BN, BK, waves
# along M and N, wave sets; checked on the host):
# - the tiles whose K range is split over their four waves: 1000^3, 1001 x 999
#   x 1000, 4001 x 67 x 320 and 70 x 4000 x 4000 hold one 64x64 tile per
#   compute unit, 1500 x 1100 x 320 and 2040 x 1000 x 1000 two (1000 = 31 *
#   32 + 8: a partial last chunk); 1501 x 1499 x 333 and 1499 x 1501 x 1000
#   one 96x96 tile, 2001 x 2047 x 77, 2046 x 2045 x 100 and 1900 x 2100 x 77
#   one 128x128; their odd widths shift the groups read at the right edge (B
#   as given) or bottom edge (A transposed) by 1, 2 or 3;
# - 60 x 12000 x 333 (under 64 rows) takes the two-set 64x64 tile, 120 x 30000
#   x 77 (under 128) the eight-wave 128x128 tile;
# - 4300^2 and 2001 x 4095 hold two or more 128x128 tiles per compute unit and
#   take the four-wave one; 300 x 257 and 37 x 45 take the 32x32 tile whose
#   slabs two single waves share; 2560 x 2530 the plain 64x64 tile.
WSPLIT = (64, 64, 32, 1, 1, 4)
WSPLIT96 = (96, 96, 32, 1, 1, 4)
WSPLIT128 = (128, 128, 16, 1, 1, 4)
KSPLIT = (64, 64, 32, 2, 2, 2)
MID = (128, 128, 32, 2, 4, 1)
RAGGED = [((5000, 3000, 333), (256, 256, 16, 4, 2, 1)), ((4300, 4300, 130), (128, 128, 16, 2, 2, 1)),
          ((3001, 2047, 4093), (192, 128, 16, 2, 2, 1)), ((2047, 3001, 4093), (128, 192, 16, 2, 2, 1)),
          ((1900, 2100, 77), WSPLIT128), ((2001, 2047, 77), WSPLIT128), ((2046, 2045, 100), WSPLIT128),
          ((1501, 1499, 333), WSPLIT96), ((1499, 1501, 1000), WSPLIT96), ((1000, 1000, 1000), WSPLIT),
          ((1001, 999, 1000), WSPLIT), ((4001, 67, 320), WSPLIT), ((70, 4000, 4000), WSPLIT),
          ((1500, 1100, 320), WSPLIT), ((2040, 1000, 1000), WSPLIT), ((60, 12000, 333), KSPLIT),
          ((120, 30000, 77), MID), ((2560, 2530, 100), (64, 64, 16, 2, 2, 1)),
          ((2900, 1910, 515), (192, 128, 16, 2, 2, 1)), ((2040, 3001, 515), (128, 192, 16, 2, 2, 1)),
          ((2001, 4095, 1001), (128, 128, 16, 2, 2, 1)), ((300, 257, 513), (32, 32, 32, 1, 1, 2)),
          ((37, 45, 77), (32, 32, 32, 1, 1, 2))]


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("shape,tile", RAGGED, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in RAGGED])
def test_edge_tiles_of_every_shape(shape, tile, pair):
    M, N, K = shape
    tA, tB = pair
    assert sg.sgemm_mfma_shape(M, N, K) == tile
    print(f"[edges] {M}x{N}x{K} tile {tile} pair {pair}", flush=True)
    opA = synth.uniform_pm1(M + 11, (M, K))
    opB = synth.uniform_pm1(N + 12, (K, N))
    C0 = synth.uniform_pm1(K + 13, (M, N))
    A, B = _stored(opA, tA), _stored(opB, tB)
    rng = np.random.default_rng(M + N)
    last_r = np.arange(max(0, M - 70), M)
    last_c = np.arange(max(0, N - 70), N)
    rows = np.concatenate([rng.integers(0, M, 2000), np.repeat(last_r, 8), rng.integers(0, M, last_c.size * 8)])
    cols = np.concatenate([rng.integers(0, N, 2000), rng.integers(0, N, last_r.size * 8), np.repeat(last_c, 8)])
    want, S = oracle.gemm_ex_entries(tA, tB, -1.25, A, B, 0.5, C0, rows, cols)
    C = gemm_ex(tA, tB, -1.25, A, B, 0.5, C0, "mfma")
    assert_within(C[rows, cols], want, S, f"{shape} {pair}")
    # The corner tile in full.
    r0, c0 = (M - 1) // tile[0] * tile[0], (N - 1) // tile[1] * tile[1]
    rr, cc = np.meshgrid(np.arange(r0, M), np.arange(c0, N), indexing="ij")
    want, S = oracle.gemm_ex_entries(tA, tB, -1.25, A, B, 0.5, C0, rr.ravel(), cc.ravel())
    assert_within(C[r0:, c0:].ravel(), want, S, f"{shape} {pair} corner tile")


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_narrow_operands(pair):
    # Widths 1..9 of the free index that is contiguous in memory (N with B as
    # given, M with A transposed): under 4 takes the general tiles, 4 and up
    # the clamped fast loop with shifted reads.
    tA, tB = pair
    print(f"[edges] narrow operands pair {pair}", flush=True)
    for w in range(1, 10):
        for (M, N) in [(w, 300), (300, w), (w, w)]:
            K = 129
            opA = synth.uniform_pm1(w + 21, (M, K))
            opB = synth.uniform_pm1(w + 22, (K, N))
            C0 = synth.uniform_pm1(w + 23, (M, N))
            A, B = _stored(opA, tA), _stored(opB, tB)
            Cref, S = oracle.gemm_ex(tA, tB, 0.75, A, B, -1.0, C0)
            C = gemm_ex(tA, tB, 0.75, A, B, -1.0, C0, "mfma")
            assert_within(C, Cref, S, f"{M}x{N}x{K} {pair}")
            Ai = synth.small_int(w + 24, (M, K))
            Bi = synth.small_int(w + 25, (K, N))
            Ci = gemm_ex(tA, tB, 1.0, _stored(Ai, tA), _stored(Bi, tB), 0.0, np.zeros((M, N), np.float32), "mfma")
            assert np.array_equal(Ci.astype(np.int64), Ai.astype(np.int64) @ Bi.astype(np.int64)), (M, N, pair)
