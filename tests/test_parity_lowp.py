"""Parity of the reduced-precision workload (bf16 / f16 operands, FP32
accumulation) with the oracle (GPU tests).

The oracle is the general-form oracle applied to the operands widened
exactly to float32 (oracle.lowp_to_float32). Products of two 16-bit values are
exact in float32, so the only rounding is the FP32 summation, and the
acceptance bound is the FP32 path's: |C - Cref| <= 1e-5 * S + 1e-6 with
S = |alpha| sum_k |op(A)_ik op(B)_kj| + |beta C0_ij|; bit-exact on small
integers.
"""

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import oracle
import synth
from oracle.check import assert_within
from tests.gpu_util import SENTINEL, gemm_lp

pytestmark = pytest.mark.gpu

PAIRS = [(False, False), (False, True), (True, False), (True, True)]
PAIR_IDS = ["nn", "nt", "tn", "tt"]
DTYPES = ["bf16", "f16"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _stored(x, trans):
    return np.ascontiguousarray(x.T) if trans else x


def _case(dtype, M, N, K, seed, dist="pm1"):
    """Stored-order-free operands: op(A) values, op(B) values (exact in
    dtype) and a float32 C0."""
    return (synth.lowp_values(seed, (M, K), dtype, dist), synth.lowp_values(seed + 1, (K, N), dtype, dist),
            synth.uniform_pm1(seed + 2, (M, N)))


def _run(dtype, tA, tB, alpha, opA, opB, beta, C0, **kw):
    """(GPU result, oracle result, error scale) for one product."""
    A = synth.to_lowp_bits(_stored(opA, tA), dtype)
    B = synth.to_lowp_bits(_stored(opB, tB), dtype)
    C = gemm_lp(dtype, tA, tB, alpha, A, B, beta, C0, **kw)
    Cref, S = oracle.gemm_ex(tA, tB, alpha, oracle.lowp_to_float32(A, dtype), oracle.lowp_to_float32(B, dtype),
                             beta, C0)
    return C, Cref, S


SHAPES = [(1, 1, 1), (5, 3, 7), (8, 8, 8), (17, 15, 17), (33, 31, 7), (65, 63, 65), (129, 127, 129),
          (255, 257, 33), (300, 1, 129), (1, 300, 129), (256, 256, 255), (520, 776, 336)]
SCALARS = [(1.0, 0.0), (-1.5, 0.75), (float(np.float32(0.3)), -2.0), (2.0, 1.0)]


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_shapes_and_scalars(dtype, pair):
    tA, tB = pair
    print(f"[lowp] shapes {dtype} {pair}", flush=True)
    for idx, (M, N, K) in enumerate(SHAPES):
        opA, opB, C0 = _case(dtype, M, N, K, 100 + 10 * idx)
        alpha, beta = SCALARS[idx % len(SCALARS)]
        C, Cref, S = _run(dtype, tA, tB, alpha, opA, opB, beta, C0)
        assert_within(C, Cref, S, f"{dtype} {pair} {M}x{N}x{K}")


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_small_integers_bit_exact(dtype, pair):
    tA, tB = pair
    print(f"[lowp] small integers {dtype} {pair}", flush=True)
    for (M, N, K) in [(300, 257, 513), (777, 555, 1001), (1024, 1024, 1024)]:
        opA, opB, _ = _case(dtype, M, N, K, 7, dist="int")
        C0 = synth.small_int(9, (M, N))
        C, _, _ = _run(dtype, tA, tB, 3.0, opA, opB, -2.0, C0)
        # Every partial sum is an integer far below 2^53, so float64 BLAS
        # gives the exact product whatever its order.
        want = 3 * (opA.astype(np.float64) @ opB.astype(np.float64)) - 2 * C0.astype(np.float64)
        assert np.array_equal(C.astype(np.float64), want), (M, N, K)


# The register-staged 64x64 tile (products too small to give every compute
# unit a larger tile, such as 1000 x 1000) walks K in slabs of 64: K on both
# sides of one to four whole slabs, with a partial one.
LP_SLAB_KS = [1, 16, 63, 64, 65, 127, 128, 129, 192, 193, 255, 261]


@pytest.mark.parametrize("K", LP_SLAB_KS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_small_tile_slab_boundaries(dtype, K):
    M = N = 1000
    # The 16-bit launch takes the largest of its 256x256, 128x128 and 64x64
    # tiles whose count reaches the compute units (256 on MI355X): 1000 x 1000
    # has 16 and 64 of the larger two, so it runs the 64x64 tile with slabs of 64.
    tiles = lambda t: -(-M // t) * -(-N // t)
    assert tiles(256) < 256 and tiles(128) < 256
    for tA, tB in PAIRS:
        print(f"[lowp] slab boundaries {dtype} {M}x{N}x{K} {(tA, tB)}", flush=True)
        opA, opB, _ = _case(dtype, M, N, K, K + 40, dist="int")
        C0 = synth.small_int(K + 41, (M, N))
        C, _, _ = _run(dtype, tA, tB, 1.0, opA, opB, 0.0, C0)
        want = opA.astype(np.float64) @ opB.astype(np.float64)
        assert np.array_equal(C.astype(np.float64), want), (M, N, K, tA, tB)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_ragged_and_large_sampled(dtype, pair):
    # The ragged shape (every edge partial, K tail) and 4096^3, checked on
    # sampled elements including the last rows and columns.
    tA, tB = pair
    for (M, N, K) in [(3001, 2047, 4093), (4096, 4096, 4096)]:
        print(f"[lowp] {M}x{N}x{K} {dtype} {pair}", flush=True)
        opA, opB, C0 = _case(dtype, M, N, K, 31, dist="pm1" if M == 3001 else "u01")
        A = synth.to_lowp_bits(_stored(opA, tA), dtype)
        B = synth.to_lowp_bits(_stored(opB, tB), dtype)
        C = gemm_lp(dtype, tA, tB, -0.5, A, B, 1.0, C0)
        rng = np.random.default_rng(M)
        rows = np.concatenate([rng.integers(0, M, 2000), np.arange(M - 40, M).repeat(10), rng.integers(0, M, 400)])
        cols = np.concatenate([rng.integers(0, N, 2000), rng.integers(0, N, 400), np.arange(N - 40, N).repeat(10)])
        want, S = oracle.gemm_ex_entries(tA, tB, -0.5, oracle.lowp_to_float32(A, dtype),
                                         oracle.lowp_to_float32(B, dtype), 1.0, C0, rows, cols)
        assert_within(C[rows, cols], want, S, f"{dtype} {pair} {M}x{N}x{K}")


def _sampled(dtype, tA, tB, M, N, K, seed, alpha=-0.5, beta=1.0, **kw):
    """Run one product and check ~5000 sampled elements (with the last rows
    and columns, and the whole bottom-right 256 x 256 tile) with the oracle."""
    opA, opB, C0 = _case(dtype, M, N, K, seed)
    A = synth.to_lowp_bits(_stored(opA, tA), dtype)
    B = synth.to_lowp_bits(_stored(opB, tB), dtype)
    C = gemm_lp(dtype, tA, tB, alpha, A, B, beta, C0, **kw)
    rng = np.random.default_rng(seed)
    r0, c0 = (M - 1) // 256 * 256, (N - 1) // 256 * 256
    rr, cc = np.meshgrid(np.arange(r0, M), np.arange(c0, N), indexing="ij")
    rows = np.concatenate([rng.integers(0, M, 2000), np.arange(M - 40, M).repeat(10), rng.integers(0, M, 400),
                           rr.ravel()])
    cols = np.concatenate([rng.integers(0, N, 2000), rng.integers(0, N, 400), np.arange(N - 40, N).repeat(10),
                           cc.ravel()])
    want, S = oracle.gemm_ex_entries(tA, tB, alpha, oracle.lowp_to_float32(A, dtype), oracle.lowp_to_float32(B, dtype),
                                     beta, C0, rows, cols)
    assert_within(C[rows, cols], want, S, f"{dtype} {(tA, tB)} {M}x{N}x{K} {kw}")


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_direct_to_lds_edges(dtype, pair):
    # Products large enough for the direct-to-LDS 256 x 256 kernel (at least
    # one tile per compute unit) with partial tiles on both edges (the free
    # index that is contiguous in memory a multiple of 8, as that kernel
    # needs) and a partial last slab of K.
    tA, tB = pair
    print(f"[lowp] direct-to-LDS edges {dtype} {pair}", flush=True)
    _sampled(dtype, tA, tB, 4000, 4104, 1000, 61)


@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_direct_to_lds_fallbacks(dtype):
    # The same tile count with one condition of the direct-to-LDS kernel
    # broken each time, so the register-staged kernel takes the product: an
    # FC extent that is not a multiple of 8, a leading dimension that is not,
    # and an operand start that is not 16-byte aligned.
    print(f"[lowp] direct-to-LDS fallbacks {dtype}", flush=True)
    _sampled(dtype, True, False, 4004, 4104, 520, 71)           # M % 8 with A transposed
    _sampled(dtype, False, False, 4096, 4100, 520, 72)          # N % 8 with B as given
    _sampled(dtype, False, True, 4096, 4096, 520, 73, ld_pad=(4, 0, 0))
    _sampled(dtype, False, False, 4096, 4096, 520, 74, offset=(0, 3, 0))


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_lp_direct_to_lds_matches_register_path_bitwise(pair):
    # Both kernels feed each lane the same k of every step of 16 and walk the
    # steps in the same order, so the same product gives the same bits
    # whichever runs: here the direct-to-LDS kernel (aligned A) against the
    # register-staged one (A starting one element into its buffer).
    tA, tB = pair
    M, N, K = 4096, 4096, 520
    print(f"[lowp] direct-to-LDS vs register path {pair}", flush=True)
    opA, opB, C0 = _case("bf16", M, N, K, 91)
    A = synth.to_lowp_bits(_stored(opA, tA), "bf16")
    B = synth.to_lowp_bits(_stored(opB, tB), "bf16")
    C1 = gemm_lp("bf16", tA, tB, 0.75, A, B, -1.0, C0)
    C2 = gemm_lp("bf16", tA, tB, 0.75, A, B, -1.0, C0, offset=(1, 0, 0))
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


@pytest.mark.parametrize("pair", [(False, False), (True, True)], ids=["nn", "tt"])
def test_lp_direct_to_lds_small_integers_bit_exact(pair):
    # Small integers: every partial sum is an integer below 2^24, so the
    # result is exact whatever the summation order; checked against float64
    # matrix products.
    tA, tB = pair
    M, N, K = 4096, 4096, 1024
    print(f"[lowp] direct-to-LDS small integers {pair}", flush=True)
    opA = synth.lowp_values(81, (M, K), "bf16", "int")
    opB = synth.lowp_values(82, (K, N), "bf16", "int")
    A = synth.to_lowp_bits(_stored(opA, tA), "bf16")
    B = synth.to_lowp_bits(_stored(opB, tB), "bf16")
    C = gemm_lp("bf16", tA, tB, 1.0, A, B, 0.0, np.zeros((M, N), np.float32))
    want = opA.astype(np.float64) @ opB.astype(np.float64)
    assert np.array_equal(C.astype(np.float64), want)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_lp_direct_to_lds_padded_c(pair):
    # The direct-to-LDS kernel's epilogue (C staged through LDS, stored four
    # columns at a time) into a C whose rows are padded to an odd length and
    # whose start is 12 bytes past a 16-byte boundary; A and B keep what that
    # kernel needs (16-byte aligned, leading dimensions padded by 8), and the
    # product is ragged on both edges. Equal bit for bit to the packed run,
    # and nothing outside C's window changes.
    tA, tB = pair
    M, N, K = 4000, 4104, 520
    print(f"[lowp] direct-to-LDS padded C {pair}", flush=True)
    opA, opB, C0 = _case("bf16", M, N, K, 95)
    A = synth.to_lowp_bits(_stored(opA, tA), "bf16")
    B = synth.to_lowp_bits(_stored(opB, tB), "bf16")
    packed = gemm_lp("bf16", tA, tB, 1.5, A, B, -0.25, C0)
    C, cbuf, ldc, off = gemm_lp("bf16", tA, tB, 1.5, A, B, -0.25, C0, ld_pad=(8, 8, 9), offset=(0, 0, 3),
                                return_buffer=True)
    assert np.array_equal(C.view(np.uint32), packed.view(np.uint32)), pair
    mask = np.ones(cbuf.shape, bool)
    mask[(off + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]).ravel()] = False
    assert (cbuf[mask] == SENTINEL).all()


@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_narrow_operands(dtype):
    # Row-contiguous free extents 1..12: under 8 the one-per-element kernel,
    # from 8 the matrix-core kernel with clamped, shifted edge reads.
    print(f"[lowp] narrow {dtype}", flush=True)
    for tA, tB in PAIRS:
        for w in range(1, 13):
            for (M, N) in [(w, 300), (300, w)]:
                opA, opB, C0 = _case(dtype, M, N, 47, w)
                C, Cref, S = _run(dtype, tA, tB, 1.25, opA, opB, 0.5, C0)
                assert_within(C, Cref, S, f"{dtype} {(tA, tB)} {M}x{N}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_strided_views_and_misaligned_starts(dtype):
    # Operands inside larger buffers (NaN encodings in the padding) at odd
    # element offsets (2-byte aligned starts), C updated in place: every run
    # equals the packed run bit for bit, and nothing outside C changes.
    M, N, K = 150, 260, 333
    for tA, tB in PAIRS:
        print(f"[lowp] strided {dtype} {(tA, tB)}", flush=True)
        opA, opB, C0 = _case(dtype, M, N, K, 500)
        packed, Cref, S = _run(dtype, tA, tB, -0.75, opA, opB, 0.5, C0)
        assert_within(packed, Cref, S, "packed")
        for pads, offs in [((4, 4, 4), (0, 0, 0)), ((3, 5, 7), (0, 0, 0)), ((0, 0, 0), (1, 3, 5)),
                           ((5, 1, 9), (3, 1, 2))]:
            A = synth.to_lowp_bits(_stored(opA, tA), dtype)
            B = synth.to_lowp_bits(_stored(opB, tB), dtype)
            C, cbuf, ldc, off = gemm_lp(dtype, tA, tB, -0.75, A, B, 0.5, C0, ld_pad=pads, offset=offs,
                                        return_buffer=True)
            assert np.array_equal(C, packed), (tA, tB, pads, offs)
            mask = np.ones(cbuf.shape, bool)
            mask[(off + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]).ravel()] = False
            assert (cbuf[mask] == SENTINEL).all()


@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_blas_read_rules_and_determinism(dtype):
    print(f"[lowp] read rules {dtype}", flush=True)
    M, N, K = 130, 140, 150
    opA, opB, C0 = _case(dtype, M, N, K, 600)
    # beta = 0: NaN in C is not read.
    C, Cref, S = _run(dtype, False, False, 1.0, opA, opB, 0.0, np.full((M, N), np.nan, np.float32))
    assert_within(C, oracle.gemm_ex(False, False, 1.0, opA, opB, 0.0, None)[0], S, "beta 0")
    # alpha = 0: NaN encodings in A and B are not read.
    nanA = np.full((M, K), 0x7FFF, np.uint16)
    nanB = np.full((K, N), 0x7FFF, np.uint16)
    C = gemm_lp(dtype, False, False, 0.0, nanA, nanB, -0.5, C0)
    assert np.array_equal(C, np.float32(-0.5) * C0)
    # Repeated runs are bit-identical.
    first = _run(dtype, True, False, 1.0, opA, opB, 0.0, C0)[0]
    for _ in range(3):
        assert np.array_equal(_run(dtype, True, False, 1.0, opA, opB, 0.0, C0)[0], first)


def test_lp_tensor_api():
    print("[lowp] tensor API", flush=True)
    M, N, K = 300, 200, 100
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        X = synth.lowp_values(700, (K, M), dt)      # op(A) = X^T
        Y = synth.lowp_values(701, (K, N), dt)
        dX = torch.from_numpy(X).to(tdt).cuda()
        dY = torch.from_numpy(Y).to(tdt).cuda()
        C = sg.gemm(dX.t(), dY).cpu().numpy()
        Cref, S = oracle.gemm_ex(True, False, 1.0, X, Y, 0.0, None)
        assert_within(C, Cref, S, f"tensor API {dt}")


# The 192 x 128 register-staged tile (A stored M x K: the NN and NT pairs).
# The launch takes it in place of 128 x 128 where its rounds of one tile per
# compute unit cover less area: 3001 x 2047 has 16 x 16 of them against
# 24 x 16 of 128 x 128 (and under 256 of the 256 x 256 tiles).
def _takes_wide_lp(M, N, tA):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = lambda bm, bn: -(-M // bm) * -(-N // bn)
    rounds = lambda t: -(-t // cus)
    return (not tA and tiles(256, 256) < cus and tiles(128, 128) >= cus and
            rounds(tiles(192, 128)) * 192 * 128 < rounds(tiles(128, 128)) * 128 * 128)


WIDE_KS = [1, 16, 63, 64, 65, 129, 192, 255]


@pytest.mark.parametrize("pair", [(False, False), (False, True)], ids=["nn", "nt"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_wide_tile_slab_boundaries(dtype, pair):
    # Small integers over K on both sides of one to four slabs of 64, every
    # edge partial: the exact integer product over the whole of C.
    tA, tB = pair
    M, N = 3001, 2047
    assert _takes_wide_lp(M, N, tA)
    for K in WIDE_KS:
        print(f"[lowp] 192x128 tile {dtype} {M}x{N}x{K} {pair}", flush=True)
        opA, opB, _ = _case(dtype, M, N, K, K + 50, dist="int")
        C, _, _ = _run(dtype, tA, tB, 1.0, opA, opB, 0.0, np.zeros((M, N), np.float32))
        want = opA.astype(np.float64) @ opB.astype(np.float64)
        assert np.array_equal(C.astype(np.float64), want), (M, N, K, pair)


@pytest.mark.parametrize("pair", [(False, False), (False, True)], ids=["nn", "nt"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_lp_wide_tile_padded_window(dtype, pair):
    # Padded, misaligned operands and C (the register-staged tile reads and
    # writes at any 2- and 4-byte alignment), alpha and beta, a partial last
    # slab; sampled against the oracle, and nothing outside C's window changes.
    tA, tB = pair
    M, N, K = 2990, 2041, 515
    assert _takes_wide_lp(M, N, tA)
    print(f"[lowp] 192x128 tile padded {dtype} {pair}", flush=True)
    opA, opB, C0 = _case(dtype, M, N, K, 101)
    A = synth.to_lowp_bits(_stored(opA, tA), dtype)
    B = synth.to_lowp_bits(_stored(opB, tB), dtype)
    C, cbuf, ldc, off = gemm_lp(dtype, tA, tB, -1.25, A, B, 0.5, C0, ld_pad=(3, 5, 7), offset=(1, 2, 3),
                                return_buffer=True)
    rng = np.random.default_rng(7)
    rows = np.concatenate([rng.integers(0, M, 3000), np.arange(M - 64, M).repeat(8)])
    cols = np.concatenate([rng.integers(0, N, 3000), np.arange(N - 64, N).repeat(8)])
    want, S = oracle.gemm_ex_entries(tA, tB, -1.25, oracle.lowp_to_float32(A, dtype),
                                     oracle.lowp_to_float32(B, dtype), 0.5, C0, rows, cols)
    assert_within(C[rows, cols], want, S, f"{dtype} {pair} 192x128 padded")
    mask = np.ones(cbuf.shape, bool)
    mask[(off + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]).ravel()] = False
    assert (cbuf[mask] == SENTINEL).all()


@pytest.mark.parametrize("pair", [(False, False), (False, True)], ids=["nn", "nt"])
def test_lp_wide_tile_same_bits_as_other_tiles(pair):
    # Every register-staged tile walks k in the same steps of 16 in the same
    # order, so the top-left 1000 x 1000 of a 192 x 128-tile product equals
    # the 1000 x 1000 product (64 x 64 tiles) bit for bit.
    tA, tB = pair
    M, N, K = 3001, 2047, 777
    assert _takes_wide_lp(M, N, tA) and not _takes_wide_lp(1000, 1000, tA)
    print(f"[lowp] 192x128 tile vs 64x64 tile bits {pair}", flush=True)
    opA, opB, C0 = _case("bf16", M, N, K, 111)
    full = gemm_lp("bf16", tA, tB, 1.0, synth.to_lowp_bits(_stored(opA, tA), "bf16"),
                   synth.to_lowp_bits(_stored(opB, tB), "bf16"), 0.0, C0)
    sub = gemm_lp("bf16", tA, tB, 1.0, synth.to_lowp_bits(_stored(np.ascontiguousarray(opA[:1000]), tA), "bf16"),
                  synth.to_lowp_bits(_stored(np.ascontiguousarray(opB[:, :1000]), tB), "bf16"), 0.0,
                  np.ascontiguousarray(C0[:1000, :1000]))
    assert np.array_equal(full[:1000, :1000].view(np.uint32), sub.view(np.uint32))
