"""Seeded random products against the oracle (GPU tests).

The shape lists of the other parity tests are chosen by hand. These draw the
sizes, the transpose pair, alpha and beta, leading-dimension padding and start
offsets from a seeded generator, so tile choices and edge combinations that no
list names are covered too. Sizes are log-uniform in [1, 3000] (FP32) or
[1, 2500] (16-bit), a quarter of them within one of a power of two from 64 to
2048. Every case checks 600
random entries plus the whole last row and column against the oracle, through
sgemm_ex (variant best; every third case through sgemm_ex_ws with a workspace)
for FP32 and through sgemm_lp for bf16 and f16; a third set runs the naive,
tiled and register-blocked rungs in turn, and a fourth draws large products
(M and N in [1700, 4400]) for the large tiles of both paths.
"""

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import oracle
import synth
from oracle.check import assert_within
from tests.gpu_util import gemm_ex, gemm_lp

pytestmark = pytest.mark.gpu

SCALARS = [(1.0, 0.0), (-0.5, 1.0), (2.0, -0.25), (0.75, 0.5)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


@pytest.fixture(scope="module")
def workspace():
    return torch.full((160 << 20,), 0xFF, dtype=torch.uint8, device="cuda")


def _cases(seed: int, n: int, largest: int):
    rng = np.random.default_rng(seed)

    def size():
        if rng.random() < 0.25:
            return int(rng.choice([64, 128, 256, 512, 1024, 2048])) + int(rng.integers(-1, 2))
        return max(1, int(np.exp(rng.uniform(0.0, np.log(largest)))))

    out = []
    for i in range(n):
        M, N, K = size(), size(), size()
        tA, tB = bool(rng.integers(2)), bool(rng.integers(2))
        alpha, beta = SCALARS[int(rng.integers(len(SCALARS)))]
        pads = tuple(int(x) for x in rng.integers(0, 6, 3)) if rng.random() < 0.5 else (0, 0, 0)
        offs = tuple(int(x) for x in rng.integers(0, 4, 3)) if rng.random() < 0.3 else (0, 0, 0)
        out.append((i, M, N, K, tA, tB, alpha, beta, pads, offs))
    return out


def _stored(x, trans):
    return np.ascontiguousarray(x.T) if trans else x


def _sample(M, N, seed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([rng.integers(0, M, 600), np.full(N, M - 1), np.arange(M)])
    cols = np.concatenate([rng.integers(0, N, 600), np.arange(N), np.full(M, N - 1)])
    return rows, cols


FP32_CASES = _cases(2024, 160, 3000)
LOWP_CASES = _cases(4048, 96, 2500)


def _id(c):
    i, M, N, K, tA, tB, *_ = c
    return f"{i}-{M}x{N}x{K}-{'t' if tA else 'n'}{'t' if tB else 'n'}"


@pytest.mark.parametrize("case", FP32_CASES, ids=_id)
def test_random_fp32(case, workspace):
    i, M, N, K, tA, tB, alpha, beta, pads, offs = case
    print(f"[random] fp32 {_id(case)} alpha {alpha} beta {beta} pads {pads} offsets {offs}", flush=True)
    opA = synth.uniform_pm1(3 * i + 1, (M, K))
    opB = synth.uniform_pm1(3 * i + 2, (K, N))
    C0 = synth.uniform_pm1(3 * i + 3, (M, N))
    A, B = _stored(opA, tA), _stored(opB, tB)
    ws = workspace if i % 3 == 0 else None
    C = gemm_ex(tA, tB, alpha, A, B, beta, C0, "best", ld_pad=pads, offset=offs, workspace=ws)
    rows, cols = _sample(M, N, i)
    want, S = oracle.gemm_ex_entries(tA, tB, alpha, A, B, beta, C0, rows, cols)
    assert_within(C[rows, cols], want, S, _id(case))


@pytest.mark.parametrize("case", LOWP_CASES, ids=_id)
def test_random_lowp(case):
    i, M, N, K, tA, tB, alpha, beta, pads, offs = case
    dtype = "bf16" if i % 2 == 0 else "f16"
    print(f"[random] {dtype} {_id(case)} alpha {alpha} beta {beta} pads {pads} offsets {offs}", flush=True)
    opA = synth.lowp_values(3 * i + 101, (M, K), dtype, "pm1")
    opB = synth.lowp_values(3 * i + 102, (K, N), dtype, "pm1")
    C0 = synth.uniform_pm1(3 * i + 103, (M, N))
    A = synth.to_lowp_bits(_stored(opA, tA), dtype)
    B = synth.to_lowp_bits(_stored(opB, tB), dtype)
    C = gemm_lp(dtype, tA, tB, alpha, A, B, beta, C0, ld_pad=pads, offset=offs)
    rows, cols = _sample(M, N, i)
    want, S = oracle.gemm_ex_entries(tA, tB, alpha, oracle.lowp_to_float32(A, dtype), oracle.lowp_to_float32(B, dtype),
                                     beta, C0, rows, cols)
    assert_within(C[rows, cols], want, S, f"{dtype} {_id(case)}")


# Large products: M and N uniform in [1700, 4400], K log-uniform in [1, 3000],
# so that the large tiles (256 x 256, 192 x 128, 128 x 192, both 128 x 128
# tiles and the 16-bit ones) run with every edge combination and transpose
# pair.
def _large_cases(seed: int, n: int):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N = (int(x) for x in rng.integers(1700, 4401, 2))
        K = max(1, int(np.exp(rng.uniform(0.0, np.log(3000)))))
        tA, tB = bool(rng.integers(2)), bool(rng.integers(2))
        alpha, beta = SCALARS[int(rng.integers(len(SCALARS)))]
        pads = tuple(int(x) for x in rng.integers(0, 6, 3)) if rng.random() < 0.5 else (0, 0, 0)
        offs = tuple(int(x) for x in rng.integers(0, 4, 3)) if rng.random() < 0.3 else (0, 0, 0)
        out.append((i, M, N, K, tA, tB, alpha, beta, pads, offs))
    return out


LARGE_CASES = _large_cases(8096, 24)


@pytest.mark.parametrize("case", LARGE_CASES, ids=_id)
def test_random_large_fp32(case, workspace):
    i, M, N, K, tA, tB, alpha, beta, pads, offs = case
    print(f"[random] large fp32 {_id(case)} tile {sg.sgemm_mfma_tile(M, N, K)} alpha {alpha} beta {beta} pads {pads} "
          f"offsets {offs}", flush=True)
    opA = synth.uniform_pm1(3 * i + 301, (M, K))
    opB = synth.uniform_pm1(3 * i + 302, (K, N))
    C0 = synth.uniform_pm1(3 * i + 303, (M, N))
    A, B = _stored(opA, tA), _stored(opB, tB)
    ws = workspace if i % 3 == 0 else None
    C = gemm_ex(tA, tB, alpha, A, B, beta, C0, "best", ld_pad=pads, offset=offs, workspace=ws)
    rows, cols = _sample(M, N, i)
    want, S = oracle.gemm_ex_entries(tA, tB, alpha, A, B, beta, C0, rows, cols)
    assert_within(C[rows, cols], want, S, _id(case))


@pytest.mark.parametrize("case", LARGE_CASES, ids=_id)
def test_random_large_lowp(case):
    i, M, N, K, tA, tB, alpha, beta, pads, offs = case
    dtype = "bf16" if i % 2 == 0 else "f16"
    print(f"[random] large {dtype} {_id(case)} alpha {alpha} beta {beta} pads {pads} offsets {offs}", flush=True)
    opA = synth.lowp_values(3 * i + 401, (M, K), dtype, "pm1")
    opB = synth.lowp_values(3 * i + 402, (K, N), dtype, "pm1")
    C0 = synth.uniform_pm1(3 * i + 403, (M, N))
    A = synth.to_lowp_bits(_stored(opA, tA), dtype)
    B = synth.to_lowp_bits(_stored(opB, tB), dtype)
    C = gemm_lp(dtype, tA, tB, alpha, A, B, beta, C0, ld_pad=pads, offset=offs)
    rows, cols = _sample(M, N, i)
    want, S = oracle.gemm_ex_entries(tA, tB, alpha, oracle.lowp_to_float32(A, dtype), oracle.lowp_to_float32(B, dtype),
                                     beta, C0, rows, cols)
    assert_within(C[rows, cols], want, S, f"{dtype} {_id(case)}")


RUNG_CASES = _cases(6072, 48, 1500)


@pytest.mark.parametrize("case", RUNG_CASES, ids=_id)
def test_random_every_rung(case):
    # The same draws for the naive, tiled and register-blocked rungs, one per
    # case in turn (the matrix-core rung is the "best" above).
    i, M, N, K, tA, tB, alpha, beta, pads, offs = case
    variant = ("naive", "tiled", "regblock")[i % 3]
    print(f"[random] {variant} {_id(case)} alpha {alpha} beta {beta} pads {pads} offsets {offs}", flush=True)
    opA = synth.uniform_pm1(3 * i + 201, (M, K))
    opB = synth.uniform_pm1(3 * i + 202, (K, N))
    C0 = synth.uniform_pm1(3 * i + 203, (M, N))
    A, B = _stored(opA, tA), _stored(opB, tB)
    C = gemm_ex(tA, tB, alpha, A, B, beta, C0, variant, ld_pad=pads, offset=offs)
    rows, cols = _sample(M, N, i)
    want, S = oracle.gemm_ex_entries(tA, tB, alpha, A, B, beta, C0, rows, cols)
    assert_within(C[rows, cols], want, S, f"{variant} {_id(case)}")
