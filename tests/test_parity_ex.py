"""Parity of the general form C = alpha * op(A) * op(B) + beta * C with the
CPU oracle, for every kernel variant and transpose pair (GPU tests).

Acceptance (per element): |C - Cref| <= 1e-5 * S + 1e-6 with Cref and
S = |alpha| sum_k |op(A)_ik op(B)_kj| + |beta C0_ij| from the oracle in
double; bit-exact where every intermediate is exact (small integers, integer
alpha and beta).
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

VARIANTS = ["naive", "tiled", "regblock", "mfma"]
PAIRS = [(False, False), (False, True), (True, False), (True, True)]
PAIR_IDS = ["nn", "nt", "tn", "tt"]
F32 = lambda x: float(np.float32(x))  # noqa: E731  (scalars as the C ABI receives them)
SCALARS = [(1.0, 0.0), (-1.5, 0.75), (F32(0.3), -2.0), (2.0, 1.0)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _announce(msg):
    print(f"[parity-ex] {msg}", flush=True)


def _stored(x, trans):
    return np.ascontiguousarray(x.T) if trans else x


def _case(M, N, K, seed):
    opA = synth.uniform_pm1(seed, (M, K))
    opB = synth.uniform_pm1(seed + 1, (K, N))
    C0 = synth.uniform_pm1(seed + 2, (M, N))
    return opA, opB, C0


_REF = {}


def _reference(key, tA, tB, alpha, A, B, beta, C0):
    """Oracle result of one case, cached across variants."""
    k = (key, tA, tB, alpha, beta)
    if k not in _REF:
        _REF[k] = oracle.gemm_ex(tA, tB, alpha, A, B, beta, C0)
    return _REF[k]


SHAPES = [(1, 1, 1), (5, 3, 7), (17, 15, 17), (33, 31, 7), (65, 63, 65), (129, 127, 129),
          (255, 257, 33), (300, 1, 129), (1, 300, 129), (256, 256, 255), (520, 776, 336)]


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("variant", VARIANTS + ["best"])
def test_ex_shapes_and_scalars(variant, pair):
    tA, tB = pair
    _announce(f"shapes variant {variant} pair {pair}")
    for idx, (M, N, K) in enumerate(SHAPES):
        opA, opB, C0 = _case(M, N, K, 1000 + idx * 10)
        A, B = _stored(opA, tA), _stored(opB, tB)
        alpha, beta = SCALARS[idx % len(SCALARS)]
        Cref, S = _reference((M, N, K), tA, tB, alpha, A, B, beta, C0)
        C = gemm_ex(tA, tB, alpha, A, B, beta, C0, variant)
        assert_within(C, Cref, S, f"{variant} {pair} {M}x{N}x{K} alpha={alpha} beta={beta}")


# Interior tiles plus bottom and right strips, partial K slabs, all three
# interior tile sizes of the matrix-core path.
SPLIT = [(1000, 1000, 1000), (384, 512, 20), (129, 260, 4100), (2048, 1280, 1028), (4100, 4100, 40)]


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_ex_mfma_interior_and_strips(pair):
    tA, tB = pair
    _announce(f"mfma split pair {pair}")
    for idx, (M, N, K) in enumerate(SPLIT):
        opA, opB, C0 = _case(M, N, K, 2000 + idx * 10)
        A, B = _stored(opA, tA), _stored(opB, tB)
        rng = np.random.default_rng(idx)
        rows, cols = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
        rows[:4], cols[:4] = [0, M - 1, 0, M - 1], [0, 0, N - 1, N - 1]
        want, S = oracle.gemm_ex_entries(tA, tB, 0.5, A, B, -1.0, C0, rows, cols)
        C = gemm_ex(tA, tB, 0.5, A, B, -1.0, C0, "mfma")
        assert_within(C[rows, cols], want, S, f"mfma {pair} {M}x{N}x{K}")


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("variant", VARIANTS)
def test_ex_small_integers_bit_exact(variant, pair):
    # Entries in [-8, 8], alpha = 3, beta = -2: every partial sum, alpha * s,
    # beta * c and their sum are integers below 2^24, so the result is exact
    # whatever the order.
    tA, tB = pair
    _announce(f"small integers variant {variant} pair {pair}")
    for (M, N, K) in [(300, 257, 513), (1024, 1024, 1024)]:
        opA = synth.small_int(M + 1, (M, K))
        opB = synth.small_int(N + 2, (K, N))
        C0 = synth.small_int(K + 3, (M, N))
        A, B = _stored(opA, tA), _stored(opB, tB)
        want = 3 * (opA.astype(np.int64) @ opB.astype(np.int64)) - 2 * C0.astype(np.int64)
        C = gemm_ex(tA, tB, 3.0, A, B, -2.0, C0, variant)
        assert np.array_equal(C.astype(np.int64), want), (M, N, K)


@pytest.mark.parametrize("pair", PAIRS[1:], ids=PAIR_IDS[1:])
@pytest.mark.parametrize("variant", VARIANTS)
def test_ex_transposes_keep_the_summation_order(variant, pair):
    # Every variant sums each element in the same k order whichever way the
    # operands are stored, so with alpha = 1 and beta = 0 the transposed runs
    # equal the plain run bit for bit (the plain run is checked against the
    # oracle elsewhere, here on the ragged shapes too).
    tA, tB = pair
    _announce(f"transposes vs plain variant {variant} pair {pair}")
    for (M, N, K) in [(1000, 1100, 1300), (129, 260, 4100), (3001, 2047, 4093)]:
        if variant == "naive" and M * N * K > 2e9:
            continue
        opA, opB = synth.operands(M, N, K, "pm1", seed_a=M, seed_b=N)
        plain = gemm(opA, opB, variant)
        C = gemm_ex(tA, tB, 1.0, _stored(opA, tA), _stored(opB, tB), 0.0,
                    np.zeros((M, N), np.float32), variant)
        assert np.array_equal(C, plain), (M, N, K)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_ex_headline_size_sampled(pair):
    # 4096^3 as the benchmark runs it (best variant), with alpha and beta:
    # 2048 sampled elements against the oracle, computed one by one.
    tA, tB = pair
    _announce(f"4096^3 sampled pair {pair}")
    A0, B0 = synth.operands(4096, 4096, 4096, "u01")
    C0 = synth.uniform_pm1(77, (4096, 4096))
    A, B = _stored(A0, tA), _stored(B0, tB)
    rng = np.random.default_rng(5)
    rows, cols = rng.integers(0, 4096, 2048), rng.integers(0, 4096, 2048)
    want, S = oracle.gemm_ex_entries(tA, tB, -0.5, A, B, 1.0, C0, rows, cols)
    C = gemm_ex(tA, tB, -0.5, A, B, 1.0, C0, "best")
    assert_within(C[rows, cols], want, S, f"4096^3 {pair}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_ex_beta_zero_never_reads_C(variant):
    _announce(f"beta = 0 with NaN in C, variant {variant}")
    opA, opB, _ = _case(130, 140, 150, 3000)
    C0 = np.full((130, 140), np.nan, np.float32)
    for tA, tB in PAIRS:
        A, B = _stored(opA, tA), _stored(opB, tB)
        Cref, S = oracle.gemm_ex(tA, tB, 1.25, A, B, 0.0, None)
        C = gemm_ex(tA, tB, 1.25, A, B, 0.0, C0, variant)
        assert_within(C, Cref, S, f"{variant} {(tA, tB)}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_ex_alpha_zero_or_empty_sum_only_scales_C(variant):
    _announce(f"alpha = 0 / K = 0, variant {variant}")
    M, N = 70, 90
    C0 = synth.uniform_pm1(3100, (M, N))
    nanA = np.full((M, 50), np.nan, np.float32)
    nanB = np.full((50, N), np.nan, np.float32)
    for beta in (-0.5, 0.0, 1.0):
        Cref, S = oracle.gemm_ex(False, False, 0.0, nanA, nanB, beta, C0)
        C = gemm_ex(False, False, 0.0, nanA, nanB, beta, C0, variant)
        assert_within(C, Cref, S, f"alpha=0 beta={beta}")
        if beta == 1.0:
            assert np.array_equal(C, C0)          # nothing launched, C untouched
        if beta == 0.0:
            assert not C.any()
    empty_A, empty_B = np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32)
    C = gemm_ex(False, False, 1.0, empty_A, empty_B, 2.0, C0, variant)
    assert np.array_equal(C, 2.0 * C0)            # doubling is exact
    C = gemm_ex(False, False, 1.0, empty_A, empty_B, 0.0, np.full((M, N), np.nan, np.float32), variant)
    assert np.array_equal(C, np.zeros((M, N), np.float32))


@pytest.mark.parametrize("variant", VARIANTS)
def test_ex_strided_views_and_misaligned_starts(variant):
    # Stored operands inside larger buffers (NaN padding), misaligned starts,
    # C updated in place with beta != 0: each run must equal the packed run
    # bit for bit, and nothing outside C's window may change.
    M, N, K = 150, 260, 333
    opA, opB, C0 = _case(M, N, K, 4000)
    for tA, tB in PAIRS:
        _announce(f"strided views variant {variant} pair {(tA, tB)}")
        A, B = _stored(opA, tA), _stored(opB, tB)
        packed = gemm_ex(tA, tB, -0.75, A, B, 0.5, C0, variant)
        Cref, S = oracle.gemm_ex(tA, tB, -0.75, A, B, 0.5, C0)
        assert_within(packed, Cref, S, f"{variant} packed {(tA, tB)}")
        for pads, offs in [((4, 4, 4), (0, 0, 0)), ((3, 5, 7), (0, 0, 0)), ((0, 0, 0), (1, 2, 3)),
                           ((5, 1, 9), (3, 1, 2))]:
            C, cbuf, ldc, off = gemm_ex(tA, tB, -0.75, A, B, 0.5, C0, variant, ld_pad=pads, offset=offs,
                                        return_buffer=True)
            assert np.array_equal(C, packed), (tA, tB, pads, offs)
            mask = np.ones(cbuf.shape, bool)
            idx = off + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
            mask[idx.ravel()] = False
            assert (cbuf[mask] == SENTINEL).all(), (tA, tB, pads, offs)


def test_tensor_api_takes_transposed_views():
    _announce("tensor API with transposed views")
    M, N, K = 300, 200, 100
    X = synth.uniform_pm1(5000, (K, M))       # op(A) = X^T
    Y = synth.uniform_pm1(5001, (N, K))       # op(B) = Y^T
    C0 = synth.uniform_pm1(5002, (M, N))
    dX, dY = torch.from_numpy(X).cuda(), torch.from_numpy(Y).cuda()
    dC = torch.from_numpy(C0).cuda()
    out = sg.gemm(dX.t(), dY.t(), dC, alpha=2.0, beta=-1.0)
    assert out is dC
    Cref, S = oracle.gemm_ex(True, True, 2.0, X, Y, -1.0, C0)
    assert_within(dC.cpu().numpy(), Cref, S, "gemm on views")
    C2 = sg.matmul(dX.t(), dY.t()).cpu().numpy()
    Cref2, S2 = oracle.gemm_ex(True, True, 1.0, X, Y, 0.0, None)
    assert_within(C2, Cref2, S2, "matmul on views")
