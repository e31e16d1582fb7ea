"""Pins of the CPU oracle against things other than itself (host only).

The pages print no element of any product, so the oracle is pinned by exact
arithmetic and closed forms:

* exact rational brute force (Python integers) on tiny shapes, where the
  oracle's double sums are themselves exact;
* an exact integer library product (numpy int64 matmul) on small-integer
  inputs at mid sizes;
* identity, permutation, all-ones, diagonal and outer-product closed forms;
* the whole-matrix checksum identity sum_ij C_ij = sum_k colsum_A(k) *
  rowsum_B(k), evaluated exactly in Python integers;
* numpy's float64 product as a second library routine at mid sizes;
* leading-dimension handling (padding filled with NaN must never be read).
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GRID = {"u01": 24, "pm1": 23}          # inputs are integers times 2**-GRID


@pytest.fixture
def lib():
    """The oracle under test (the mutation tests pass planted-mistake builds)."""
    return oracle.load()


def _ints(x: np.ndarray, dist: str):
    """The exact integer numerators of a grid-valued float32 matrix."""
    v = x.astype(np.float64) * 2.0**GRID[dist]
    assert np.array_equal(v, np.round(v))
    return v.astype(np.int64)


def _exact_product(A, B, dist):
    """Exact C and S as Fractions, by brute force over Python integers."""
    a, b = _ints(A, dist).tolist(), _ints(B, dist).tolist()
    M, K = A.shape
    N = B.shape[1]
    scale = Fraction(1, 2 ** (2 * GRID[dist]))
    C = [[Fraction(sum(a[i][k] * b[k][j] for k in range(K))) * scale
          for j in range(N)] for i in range(M)]
    S = [[Fraction(sum(abs(a[i][k] * b[k][j]) for k in range(K))) * scale
          for j in range(N)] for i in range(M)]
    return C, S


TINY = [(1, 1, 1), (1, 9, 1), (9, 1, 1), (1, 1, 9), (2, 3, 4), (3, 2, 5),
        (5, 7, 3), (7, 5, 9), (8, 8, 8), (9, 9, 9), (4, 9, 16), (6, 3, 13)]


@pytest.mark.parametrize("dist", ["u01", "pm1"])
@pytest.mark.parametrize("M,N,K", TINY)
def test_exact_brute_force_tiny(M, N, K, dist, lib):
    # With K <= 16 every partial sum needs at most 52 significant bits, so the
    # oracle's double result must equal the exact rational value bit for bit.
    A, B = synth.operands(M, N, K, dist, seed_a=100 + M, seed_b=200 + N * K)
    C, S = oracle.gemm(A, B, with_abs=True, lib=lib)
    Cx, Sx = _exact_product(A, B, dist)
    for i in range(M):
        for j in range(N):
            assert C[i, j] == float(Cx[i][j]), (i, j)
            assert S[i, j] == float(Sx[i][j]), (i, j)


@pytest.mark.parametrize("M,N,K", [(300, 257, 513), (129, 1, 700), (1, 640, 333),
                                   (64, 64, 4096)])
def test_small_integers_equal_exact_integer_product(M, N, K, lib):
    # Entries in [-8, 8]: every partial sum is an integer below 2**53, so the
    # oracle must equal numpy's exact int64 product everywhere.
    A = synth.small_int(11, (M, K))
    B = synth.small_int(12, (K, N))
    want = A.astype(np.int64) @ B.astype(np.int64)
    C, S = oracle.gemm(A, B, with_abs=True, lib=lib)
    assert np.array_equal(C, want.astype(np.float64))
    assert np.array_equal(S, (np.abs(A).astype(np.int64) @ np.abs(B).astype(np.int64))
                          .astype(np.float64))


def test_identity_left_and_right(lib):
    B = synth.uniform_pm1(5, (37, 53))
    assert np.array_equal(oracle.gemm(np.eye(37, dtype=np.float32), B, lib=lib),
                          B.astype(np.float64))
    A = synth.uniform_pm1(6, (41, 37))
    assert np.array_equal(oracle.gemm(A, np.eye(37, dtype=np.float32), lib=lib),
                          A.astype(np.float64))


def test_permutation_reorders_rows(lib):
    rng = np.random.default_rng(3)
    perm = rng.permutation(50)
    P = np.zeros((50, 50), dtype=np.float32)
    P[np.arange(50), perm] = 1.0
    B = synth.uniform01(7, (50, 33))
    assert np.array_equal(oracle.gemm(P, B, lib=lib), B[perm].astype(np.float64))


@pytest.mark.parametrize("K", [1, 2, 7, 64, 4093])
def test_all_ones_sum_to_K(K, lib):
    A = np.ones((9, K), dtype=np.float32)
    B = np.ones((K, 11), dtype=np.float32)
    assert np.array_equal(oracle.gemm(A, B, lib=lib), np.full((9, 11), float(K)))


def test_diagonal_scaling(lib):
    d = synth.uniform_pm1(8, (40,))
    B = synth.uniform_pm1(9, (40, 23))
    C = oracle.gemm(np.diag(d).astype(np.float32), B, lib=lib)
    # One product of two float32 values is exact in double.
    assert np.array_equal(C, d.astype(np.float64)[:, None] * B.astype(np.float64))


def test_outer_product_K1(lib):
    a = synth.uniform_pm1(10, (31, 1))
    b = synth.uniform_pm1(11, (1, 29))
    assert np.array_equal(oracle.gemm(a, b, lib=lib), a.astype(np.float64) @ b.astype(np.float64))


def _exact_checksum(A, B, dist):
    a, b = _ints(A, dist), _ints(B, dist)
    return Fraction(sum(int(x) * int(y) for x, y in
                        zip(a.sum(axis=0).tolist(), b.sum(axis=1).tolist())),
                    2 ** (2 * GRID[dist]))


@pytest.mark.parametrize("dist", ["u01", "pm1"])
def test_checksum_identity_exact(dist, lib):
    # sum_ij C_ij = sum_k (sum_i A_ik)(sum_j B_kj), exact in Python integers
    # (the identity behind the whole-matrix check sum of "From 306 ms to
    # 86 ms", "How each kernel was timed"). With K = 31 every element of the
    # oracle is exact, so the correctly rounded sum of its elements (fsum)
    # must be the correctly rounded exact total.
    M, N, K = 200, 150, 31
    A, B = synth.operands(M, N, K, dist, seed_a=21, seed_b=22)
    C = oracle.gemm(A, B, lib=lib)
    assert math.fsum(C.ravel().tolist()) == float(_exact_checksum(A, B, dist))


@pytest.mark.parametrize("dist", ["u01", "pm1"])
def test_checksum_identity_long_sums(dist, lib):
    # At K = 1000 the oracle rounds; each element is within K * 2**-53 * S.
    M, N, K = 200, 150, 1000
    A, B = synth.operands(M, N, K, dist, seed_a=23, seed_b=24)
    C, S = oracle.gemm(A, B, with_abs=True, lib=lib)
    got = Fraction(math.fsum(C.ravel().tolist()))
    slack = Fraction(K * math.fsum(S.ravel().tolist())) / 2**53
    assert abs(got - _exact_checksum(A, B, dist)) <= slack


@pytest.mark.parametrize("n", [128, 257, 512])
def test_agrees_with_numpy_float64(n, lib):
    A, B = synth.operands(n, n + 3, n - 1, "pm1", seed_a=31, seed_b=32)
    C, S = oracle.gemm(A, B, with_abs=True, lib=lib)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert (np.abs(C - ref) <= 2 * n * 2.0**-53 * S).all()


def test_leading_dimensions_never_read_padding(lib):
    M, N, K = 33, 45, 27
    A, B = synth.operands(M, N, K, "pm1", seed_a=41, seed_b=42)
    Ab, Bb = synth.embed(A, K + 5), synth.embed(B, N + 3)
    C1, S1 = oracle.gemm(Ab[:, :K], Bb[:, :N], with_abs=True, lib=lib)
    C2, S2 = oracle.gemm(A, B, with_abs=True, lib=lib)
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2)
    assert not np.isnan(C1).any()


def test_entries_match_full_product_bitwise(lib):
    A, B = synth.operands(70, 90, 333, "pm1", seed_a=51, seed_b=52)
    C, S = oracle.gemm(A, B, with_abs=True, lib=lib)
    rng = np.random.default_rng(0)
    rows, cols = rng.integers(0, 70, 500), rng.integers(0, 90, 500)
    e, s = oracle.gemm_entries(A, B, rows, cols, lib=lib)
    assert np.array_equal(e, C[rows, cols]) and np.array_equal(s, S[rows, cols])
    with pytest.raises(IndexError):
        oracle.gemm_entries(A, B, [70], [0], lib=lib)


def test_empty_sum_and_empty_shapes(lib):
    A = np.zeros((4, 0), dtype=np.float32)
    B = np.zeros((0, 6), dtype=np.float32)
    assert np.array_equal(oracle.gemm(A, B, lib=lib), np.zeros((4, 6)))
    assert oracle.gemm(np.zeros((0, 5), np.float32), np.zeros((5, 3), np.float32), lib=lib).shape == (0, 3)
    assert oracle.gemm(np.zeros((2, 5), np.float32), np.zeros((5, 0), np.float32), lib=lib).shape == (2, 0)


def test_rejects_bad_operands(lib):
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((3, 4), np.float32), np.zeros((5, 2), np.float32), lib=lib)
    with pytest.raises(TypeError):
        oracle.gemm(np.zeros((3, 4)), np.zeros((4, 2)), lib=lib)
