"""Slab boundaries of the matrix-core tiles (GPU tests).

The plain 64x64 tile walks K in slabs of 16 and the two-set 64x64 and 32x32
tiles in slabs of 32, whose two halves the two wave sets share; the eight-wave 128x128 tile
walks slabs of 32 staged through two register sets, two slabs per pass of its
unrolled loop, and the four-wave 192x128, 128x192 and 128x128 tiles slabs of
16 the same way. A product runs its whole slabs through the pipelined loop
(the steady state needs three or more, the last ones run without loads) and
the partial last slab, if any, separately. The 64x64 tile whose K range is
split over its four waves deals chunks of 32 out to the waves in turn (wave
c mod 4 takes chunk c, two per pass of its loop) and gives the partial last
chunk to wave (K div 32) mod 4. These tests take K on both sides of every
such boundary, up to three whole slabs plus a partial one (up to nine chunks
for the split tile), for every transpose pair:
- small-integer operands, where every partial sum is exact and the whole of C
  must equal the integer product bit for bit;
- uniform operands with alpha and beta against the oracle on sampled outputs,
  the last row and column included.
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

WSPLIT = (64, 64, 32, 1, 1, 4)
WSPLIT96 = (96, 96, 32, 1, 1, 4)
WSPLIT128 = (128, 128, 16, 1, 1, 4)
KSPLIT = (64, 64, 32, 2, 2, 2)
MID = (128, 128, 32, 2, 4, 1)
# (M, N), the slab or chunk depth whose boundaries K walks around, and the
# kernel shape the library picks (BM, BN, BK, waves along M and N, wave
# sets): the tiles split over their waves at 1000^2 (one 64x64 tile per
# compute unit), 2048 x 1024 (two), 1500^2 (one 96x96) and 2000 x 2040 (one
# 128x128); under 64 rows the two-set 64x64 tile, under 128 the eight-wave
# 128x128 tile.
TILES = [((2560, 2530), 16, (64, 64, 16, 2, 2, 1)), ((1000, 1000), 32, WSPLIT), ((2048, 1024), 32, WSPLIT),
         ((1500, 1500), 32, WSPLIT96), ((2000, 2040), 16, WSPLIT128), ((48, 12000), 32, KSPLIT),
         ((120, 30000), 32, MID), ((3001, 2047), 16, (192, 128, 16, 2, 2, 1)),
         ((2047, 3001), 16, (128, 192, 16, 2, 2, 1)), ((2040, 4001), 16, (128, 128, 16, 2, 2, 1)),
         ((300, 257), 32, (32, 32, 32, 1, 1, 2))]
SPLIT = {WSPLIT, WSPLIT96, WSPLIT128}


def _ks(bk, shape):
    ks = {1, bk // 2, bk - 1, bk, bk + 1, 2 * bk - 1, 2 * bk, 2 * bk + 1, 3 * bk, 3 * bk + 1, 4 * bk - 1,
          4 * bk + 5, 5 * bk + 3, 6 * bk}
    if shape in SPLIT:  # the split tiles' chunks: two and more per wave, a partial ninth
        ks |= {8 * bk - 1, 8 * bk, 8 * bk + 1, 9 * bk + 7}
    return sorted(ks)


CASES = [(mn, shape, k) for mn, bk, shape in TILES for k in _ks(bk, shape)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _stored(x, trans):
    return np.ascontiguousarray(x.T) if trans else x


@pytest.mark.parametrize("mn,tile,K", CASES, ids=[f"{m}x{n}x{k}" for (m, n), _, k in CASES])
def test_slab_boundaries(mn, tile, K):
    M, N = mn
    shape = sg.sgemm_mfma_shape(M, N, K)
    assert shape == tile, shape
    for tA, tB in PAIRS:
        print(f"[slabs] {M}x{N}x{K} tile {shape} pair {(tA, tB)}", flush=True)
        Ai = synth.small_int(K + 31, (M, K))
        Bi = synth.small_int(K + 32, (K, N))
        Ci = gemm_ex(tA, tB, 1.0, _stored(Ai, tA), _stored(Bi, tB), 0.0, np.zeros((M, N), np.float32), "mfma")
        exact = Ai.astype(np.int64) @ Bi.astype(np.int64)
        assert np.array_equal(Ci.astype(np.int64), exact), (M, N, K, tA, tB)

        opA = synth.uniform_pm1(K + 33, (M, K))
        opB = synth.uniform_pm1(K + 34, (K, N))
        C0 = synth.uniform_pm1(K + 35, (M, N))
        A, B = _stored(opA, tA), _stored(opB, tB)
        C = gemm_ex(tA, tB, 0.75, A, B, -0.5, C0, "mfma")
        rng = np.random.default_rng(K)
        rows = np.concatenate([rng.integers(0, M, 1500), np.full(N, M - 1), np.arange(M)])
        cols = np.concatenate([rng.integers(0, N, 1500), np.arange(N), np.full(M, N - 1)])
        want, S = oracle.gemm_ex_entries(tA, tB, 0.75, A, B, -0.5, C0, rows, cols)
        assert_within(C[rows, cols], want, S, f"{M}x{N}x{K} {(tA, tB)}")
