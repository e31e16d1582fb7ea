"""Parity of the register-blocked rung at each of its tiles (GPU tests).

The rung keeps a block of C per work-item in registers ("From 306 ms to 86
ms", "Register blocking"; "Matrix Multiplication -- Naive to Tiled", section
07): the pages' 128 x 128 tile with 8 x 8 per work-item, and 64 x 64 (4 x 4),
32 x 32 (2 x 2) or 16 x 16 (1 x 1) tiles for products with too few of those
to occupy the device. sgemm_regblock_tile names the tile a shape takes; every case below
first checks that its shape takes the tile it is meant to cover. Each tile
must give the oracle's result within the acceptance bound, the exact integer
product on small integers, and never write outside C's window. Every
work-item sums its elements in ascending k with one fused multiply-add per
k, whatever the tile and the storage order, so the transposed pairs equal the
plain run bit for bit, and so do products that take different tiles.
"""

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import oracle
import synth
from oracle.check import assert_within
from tests.gpu_util import SENTINEL, gemm, gemm_ex

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _announce(msg):
    print(f"[regblock] {msg}", flush=True)


def _takes(M, N, tile):
    # The library's choice on this device: the compute-unit count decides it.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert sg.sgemm_regblock_tile(M, N, cus) == tile, (M, N, tile)


# Shapes per tile (slab depth BK = 8, 16, 32, 64): a whole number of tiles,
# and each side one past and one short of a tile edge, with K around the slab.
EDGES = {
    128: [(3072, 2048, 64), (3073, 2047, 65), (3071, 2049, 63), (4095, 1921, 7)],
    64: [(1024, 1024, 64), (1025, 1023, 17), (1023, 1025, 15), (960, 1087, 1)],
    32: [(384, 384, 32), (385, 383, 33), (383, 385, 31), (420, 390, 7)],
    16: [(16, 16, 64), (17, 15, 65), (15, 17, 63), (1, 1, 1), (2, 3, 5), (1, 300, 129), (300, 1, 129), (65, 33, 7),
         (128, 128, 128)],
}


@pytest.mark.parametrize("tile", [128, 64, 32, 16])
def test_tile_edges_and_window(tile):
    for (M, N, K) in EDGES[tile]:
        _takes(M, N, tile)
        _announce(f"tile {tile}: {M}x{N}x{K}")
        A, B = synth.operands(M, N, K, "pm1", seed_a=M + 7, seed_b=N + 5 * K)
        Cref, S = oracle.gemm(A, B, with_abs=True)
        C, buf, ldc, off = gemm(A, B, "regblock", ld_pad=(3, 5, 7), offset=(1, 2, 3), return_buffer=True)
        assert_within(C, Cref, S, f"regblock {M}x{N}x{K}")
        mask = np.ones(buf.shape, bool)
        for i in range(M):
            mask[off + i * ldc: off + i * ldc + N] = False
        assert (buf[mask] == SENTINEL).all(), f"regblock {M}x{N}x{K} wrote outside C"


@pytest.mark.parametrize("tile,shape", [(128, (3001, 2047, 4093)), (64, (1000, 1000, 1000)), (32, (400, 400, 513)),
                                        (16, (300, 257, 513))])
def test_small_integers_bit_exact(tile, shape):
    M, N, K = shape
    _takes(M, N, tile)
    _announce(f"tile {tile}: small integers {M}x{N}x{K}")
    A = synth.small_int(71, (M, K))
    B = synth.small_int(72, (K, N))
    assert np.array_equal(gemm(A, B, "regblock").astype(np.float64), oracle.gemm(A, B))


@pytest.mark.parametrize("tile,shape", [(128, (3001, 2047, 65)), (64, (1000, 700, 301)), (32, (420, 390, 301)),
                                        (16, (203, 170, 301))])
def test_general_form_every_pair(tile, shape):
    M, N, K = shape
    _takes(M, N, tile)
    A, B = synth.operands(M, N, K, "pm1", seed_a=21, seed_b=22)
    C0 = synth.uniform_pm1(23, (M, N))
    plain = None
    for tA in (False, True):
        for tB in (False, True):
            _announce(f"tile {tile}: general form {(tA, tB)} {M}x{N}x{K}")
            As = np.ascontiguousarray(A.T) if tA else A
            Bs = np.ascontiguousarray(B.T) if tB else B
            Cref, S = oracle.gemm_ex(tA, tB, 1.5, As, Bs, -0.75, C0)
            C = gemm_ex(tA, tB, 1.5, As, Bs, -0.75, C0, "regblock", ld_pad=(1, 2, 3), offset=(1, 0, 2))
            assert_within(C, Cref, S, f"regblock {(tA, tB)}")
            C1 = gemm_ex(tA, tB, 1.0, As, Bs, 0.0, C0, "regblock")
            if plain is None:
                plain = C1
            assert np.array_equal(C1, plain), f"regblock {(tA, tB)} differs from the plain run"


def test_tiles_sum_alike():
    # The same rows and columns from products that take different tiles: the
    # top-left 1000 x 1000 corner of 3001 x 2047 (128 x 128 tiles) equals the
    # 1000 x 1000 product (64 x 64), its 400 x 400 corner (32 x 32) and that
    # one's 300 x 257 corner (16 x 16) bit for bit, as every tile sums each
    # element in the same order.
    K = 777
    A, B = synth.operands(3001, 2047, K, "pm1", seed_a=31, seed_b=32)
    outs = {}
    for tile, (M, N) in [(128, (3001, 2047)), (64, (1000, 1000)), (32, (400, 400)), (16, (300, 257))]:
        _takes(M, N, tile)
        _announce(f"tile {tile}: {M}x{N}x{K}")
        outs[tile] = gemm(np.ascontiguousarray(A[:M]), np.ascontiguousarray(B[:, :N]), "regblock")
    assert np.array_equal(outs[128][:1000, :1000], outs[64])
    assert np.array_equal(outs[64][:400, :400], outs[32])
    assert np.array_equal(outs[32][:300, :257], outs[16])
