"""Pins of the oracle's general form C = alpha * op(A) * op(B) + beta * C
(host only).

The vendor call on "Matrix Multiplication -- Naive to Tiled", section 07,
takes alpha, beta and a transpose flag per operand (there alpha = 1, beta = 0
and both flags say "not transposed"); the pages print no value of the general
form, so it is pinned, like the plain product, by exact arithmetic:

* exact rational brute force on tiny shapes for every transpose pair, with
  alpha a power of two (then the oracle's one rounding makes its result the
  correctly rounded exact value) and with a general alpha (then it lies within
  two roundings of the exact value);
* an exact integer product (numpy int64) on small-integer inputs and integer
  alpha, beta, for every transpose pair;
* the BLAS rules for what is read: beta = 0 never reads C, alpha = 0 never
  reads A or B (NaN planted there must not show);
* leading dimensions of every operand in both storage orders (NaN padding
  that must never be read).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GRID = 23                                # pm1 entries are integers times 2**-23
PAIRS = [(False, False), (False, True), (True, False), (True, True)]


@pytest.fixture
def lib():
    return oracle.load()


def _stored(x: np.ndarray, trans: bool) -> np.ndarray:
    """The row-major array a caller passes for logical operand x when the
    operand is flagged transposed: the transpose of x, laid out row-major."""
    return np.ascontiguousarray(x.T) if trans else x


def _frac_matrix(x: np.ndarray):
    return [[Fraction(float(v)) for v in row] for row in x.tolist()]


def _exact_ex(alpha, opA, opB, beta, C):
    """alpha * opA @ opB + beta * C and its error scale, as Fractions."""
    a, b = _frac_matrix(opA), _frac_matrix(opB)
    M, K = opA.shape
    N = opB.shape[1]
    al, be = Fraction(alpha), Fraction(beta)
    c = _frac_matrix(C) if beta != 0 else None
    out, scale = [], []
    for i in range(M):
        ro, rs = [], []
        for j in range(N):
            dot = sum((a[i][k] * b[k][j] for k in range(K)), Fraction(0))
            dabs = sum((abs(a[i][k] * b[k][j]) for k in range(K)), Fraction(0))
            cterm = be * c[i][j] if c is not None else Fraction(0)
            ro.append(al * dot + cterm)
            rs.append(abs(al) * dabs + abs(cterm))
        out.append(ro)
        scale.append(rs)
    return out, scale


TINY = [(1, 1, 1), (2, 3, 4), (5, 7, 3), (7, 5, 9), (8, 8, 8), (4, 9, 16)]
# (alpha, beta, alpha is a power of two or zero)
SCALARS = [(1.0, 0.0, True), (-2.0, 1.0, True), (0.5, float(np.float32(-0.3)), True),
           (float(np.float32(0.7)), float(np.float32(1.7)), False), (0.0, -1.5, True)]


@pytest.mark.parametrize("transA,transB", PAIRS)
@pytest.mark.parametrize("M,N,K", TINY)
def test_ex_exact_brute_force_tiny(M, N, K, transA, transB, lib):
    opA = synth.uniform_pm1(300 + M, (M, K))
    opB = synth.uniform_pm1(400 + N * K, (K, N))
    C = synth.uniform_pm1(500 + M * N, (M, N))
    A, B = _stored(opA, transA), _stored(opB, transB)
    for alpha, beta, pow2 in SCALARS:
        got, S = oracle.gemm_ex(transA, transB, alpha, A, B, beta, C, lib=lib)
        want, Sx = _exact_ex(alpha, opA, opB, beta, C)
        for i in range(M):
            for j in range(N):
                if pow2:
                    # alpha * dot is exact (K <= 16 keeps dot within 52 bits),
                    # beta * c is exact (two 24-bit factors), so the one
                    # rounding of the sum gives the correctly rounded value.
                    assert got[i, j] == float(want[i][j]), (alpha, beta, i, j)
                    assert S[i, j] == float(Sx[i][j]), (alpha, beta, i, j)
                else:
                    tol = Sx[i][j] * Fraction(3, 2**53)
                    assert abs(Fraction(got[i, j]) - want[i][j]) <= tol, (alpha, beta, i, j)
                    assert abs(Fraction(S[i, j]) - Sx[i][j]) <= tol, (alpha, beta, i, j)


@pytest.mark.parametrize("transA,transB", PAIRS)
def test_ex_small_integers_exact(transA, transB, lib):
    M, N, K = 130, 97, 301
    opA = synth.small_int(21, (M, K))
    opB = synth.small_int(22, (K, N))
    C = synth.small_int(23, (M, N))
    for alpha, beta in [(3, -2), (-1, 1), (2, 0), (0, 5)]:
        got, S = oracle.gemm_ex(transA, transB, alpha, _stored(opA, transA), _stored(opB, transB),
                                beta, C, lib=lib)
        want = alpha * (opA.astype(np.int64) @ opB.astype(np.int64)) + beta * C.astype(np.int64)
        assert np.array_equal(got, want.astype(np.float64)), (alpha, beta)
        want_s = (abs(alpha) * (np.abs(opA).astype(np.int64) @ np.abs(opB).astype(np.int64))
                  + np.abs(beta * C.astype(np.int64)))
        assert np.array_equal(S, want_s.astype(np.float64)), (alpha, beta)


def test_ex_beta_zero_never_reads_C(lib):
    opA = synth.uniform_pm1(31, (40, 50))
    opB = synth.uniform_pm1(32, (50, 60))
    C = np.full((40, 60), np.nan, dtype=np.float32)
    for tA, tB in PAIRS:
        got, _ = oracle.gemm_ex(tA, tB, -1.5, _stored(opA, tA), _stored(opB, tB), 0.0, C, lib=lib)
        assert np.isfinite(got).all()
        got2, _ = oracle.gemm_ex(tA, tB, -1.5, _stored(opA, tA), _stored(opB, tB), 0.0, None, lib=lib)
        assert np.array_equal(got, got2)


def test_ex_alpha_zero_never_reads_A_or_B(lib):
    A = np.full((40, 50), np.nan, dtype=np.float32)
    B = np.full((50, 60), np.inf, dtype=np.float32)
    C = synth.uniform_pm1(33, (40, 60))
    got, S = oracle.gemm_ex(False, False, 0.0, A, B, float(np.float32(-0.3)), C, lib=lib)
    # One product of two float32 values is exact in double.
    want = float(np.float32(-0.3)) * C.astype(np.float64)
    assert np.array_equal(got, want) and np.array_equal(S, np.abs(want))


def test_ex_plain_form_is_the_plain_product(lib):
    A, B = synth.operands(70, 90, 333, "pm1", seed_a=61, seed_b=62)
    got, S = oracle.gemm_ex(False, False, 1.0, A, B, 0.0, None, lib=lib)
    ref, Sref = oracle.gemm(A, B, with_abs=True, lib=lib)
    assert np.array_equal(got, ref) and np.array_equal(S, Sref)


@pytest.mark.parametrize("transA,transB", PAIRS)
def test_ex_leading_dimensions_never_read_padding(transA, transB, lib):
    M, N, K = 33, 45, 27
    opA = synth.uniform_pm1(71, (M, K))
    opB = synth.uniform_pm1(72, (K, N))
    C = synth.uniform_pm1(73, (M, N))
    A, B = _stored(opA, transA), _stored(opB, transB)
    Ab = synth.embed(A, A.shape[1] + 5)[:, :A.shape[1]]
    Bb = synth.embed(B, B.shape[1] + 3)[:, :B.shape[1]]
    Cb = synth.embed(C, N + 7)[:, :N]
    got, S = oracle.gemm_ex(transA, transB, 0.75, Ab, Bb, -1.25, Cb, lib=lib)
    ref, Sref = oracle.gemm_ex(transA, transB, 0.75, A, B, -1.25, C, lib=lib)
    assert np.array_equal(got, ref) and np.array_equal(S, Sref)
    assert not np.isnan(got).any()


def test_ex_rejects_bad_operands(lib):
    with pytest.raises(ValueError):      # op(A) is 4 x 3, op(B) is 4 x 2
        oracle.gemm_ex(True, False, 1.0, np.zeros((3, 4), np.float32),
                       np.zeros((4, 2), np.float32), 0.0, None, lib=lib)
    with pytest.raises(ValueError):      # beta != 0 needs C
        oracle.gemm_ex(False, False, 1.0, np.zeros((3, 4), np.float32),
                       np.zeros((4, 2), np.float32), 1.0, None, lib=lib)


@pytest.mark.parametrize("transA,transB", PAIRS)
def test_ex_entries_match_full_result_bitwise(transA, transB, lib):
    M, N, K = 70, 90, 333
    opA = synth.uniform_pm1(81, (M, K))
    opB = synth.uniform_pm1(82, (K, N))
    C = synth.uniform_pm1(83, (M, N))
    A, B = _stored(opA, transA), _stored(opB, transB)
    full, S = oracle.gemm_ex(transA, transB, -0.75, A, B, 1.25, C, lib=lib)
    rng = np.random.default_rng(1)
    rows, cols = rng.integers(0, M, 400), rng.integers(0, N, 400)
    e, s = oracle.gemm_ex_entries(transA, transB, -0.75, A, B, 1.25, C, rows, cols, lib=lib)
    assert np.array_equal(e, full[rows, cols]) and np.array_equal(s, S[rows, cols])
    with pytest.raises(IndexError):
        oracle.gemm_ex_entries(transA, transB, 1.0, A, B, 0.0, None, [M], [0], lib=lib)
