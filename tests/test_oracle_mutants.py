"""The oracle's pins must catch plausible mistakes (host only).

Each case plants one mistake in a copy of ``oracle/oracle.c`` (a dropped term,
a wrong index, a transposed or mis-strided operand, float instead of double
accumulation, a lost absolute value, a sign error, a lost alpha or beta
term), builds it with gcc into a
temporary library, and runs the pin battery of ``test_oracle.py`` against it:
at least one pin must fail. Every planted mistake keeps all memory accesses in
bounds, so a mutant can only give wrong numbers, never crash the test.
"""

import os

import pytest

import oracle
from tests import test_oracle as pins
from tests import test_oracle_ex as pins_ex

with open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")) as f:
    SOURCE = f.read()

MUTANTS = {
    "drop_last_k_term": (
        "for (int64_t k = 0; k < K; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float",
        "for (int64_t k = 0; k < K - 1; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float"),
    "skip_first_k_term": (
        "for (int64_t k = 0; k < K; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float",
        "for (int64_t k = 1; k < K; ++k) {\n            const double a = (double)A[i * lda + k];\n            const float"),
    "reversed_k_in_A": (
        "const double a = (double)A[i * lda + k];\n            const float *b",
        "const double a = (double)A[i * lda + (K - 1 - k)];\n            const float *b"),
    "B_row_stride_ignores_ld": (
        "const float *b = B + k * ldb;", "const float *b = B + k * N;"),
    "A_row_stride_ignores_ld": (
        "const double a = (double)A[i * lda + k];\n            const float *b",
        "const double a = (double)A[i * K + k];\n            const float *b"),
    "float_accumulator": (
        "c[j] += a * (double)b[j];", "c[j] = (float)(c[j] + a * (double)b[j]);"),
    "subtracts_instead_of_adds": (
        "c[j] += a * (double)b[j];", "c[j] -= a * (double)b[j];"),
    "abs_sum_loses_abs": (
        "s[j] += aa * absd((double)b[j]);", "s[j] += aa * (double)b[j];"),
    "neighbour_column_of_B": (
        "c[j] += a * (double)b[j];", "c[j] += a * (double)b[j + (j + 1 < N)];"),
    "entries_transposed_B": (
        "const double b = (double)B[k * ldb + j];",
        "const double b = (double)B[(k % (j + 1)) * ldb + j];"),
    # Mistakes in the general form alpha * op(A) * op(B) + beta * C.
    "ex_drops_beta_term": ("*out = alpha * acc + c;", "*out = alpha * acc;"),
    "ex_beta_sign": ("*out = alpha * acc + c;", "*out = alpha * acc - c;"),
    "ex_ignores_alpha": ("*out = alpha * acc + c;", "*out = acc + c;"),
    "ex_C_row_stride_short": ("beta * (double)C_in[i * ldc_in + j]", "beta * (double)C_in[i * (ldc_in - (ldc_in > 1)) + j]"),
    "ex_transA_row_stride_short": ("(transA ? A[k * lda + i] :", "(transA ? A[k * (lda - (lda > 1)) + i] :"),
    "ex_transB_neighbour_k": ("B[j * ldb + k] : B[k * ldb + j]", "B[j * ldb + (k + 1) % K] : B[k * ldb + j]"),
    "ex_transA_neighbour_row": ("(transA ? A[k * lda + i] :", "(transA ? A[k * lda + (i + 1) % lda] :"),
    "ex_scale_drops_c": ("absd(alpha) * accabs + absd(c);", "absd(alpha) * accabs;"),
    "ex_entries_wrong_element": ("ex_element(transA, transB, rows[e], cols[e],",
                                 "ex_element(transA, transB, rows[e], cols[(e + 1) % n],"),
    "ex_scale_signed_alpha": ("absd(alpha) * accabs + absd(c);", "alpha * accabs + absd(c);"),
}


def _battery(lib):
    """Run every pin against ``lib``; return the names of those that failed."""
    cases = []
    for (M, N, K) in pins.TINY:
        for dist in ("u01", "pm1"):
            cases.append((pins.test_exact_brute_force_tiny,
                          dict(M=M, N=N, K=K, dist=dist)))
    cases += [
        (pins.test_small_integers_equal_exact_integer_product, dict(M=300, N=257, K=513)),
        (pins.test_identity_left_and_right, {}),
        (pins.test_permutation_reorders_rows, {}),
        (pins.test_all_ones_sum_to_K, dict(K=7)),
        (pins.test_diagonal_scaling, {}),
        (pins.test_outer_product_K1, {}),
        (pins.test_checksum_identity_exact, dict(dist="pm1")),
        (pins.test_agrees_with_numpy_float64, dict(n=128)),
        (pins.test_leading_dimensions_never_read_padding, {}),
        (pins.test_entries_match_full_product_bitwise, {}),
    ]
    for (M, N, K) in pins_ex.TINY[:4]:
        for tA, tB in pins_ex.PAIRS:
            cases.append((pins_ex.test_ex_exact_brute_force_tiny,
                          dict(M=M, N=N, K=K, transA=tA, transB=tB)))
    for tA, tB in pins_ex.PAIRS:
        cases.append((pins_ex.test_ex_small_integers_exact, dict(transA=tA, transB=tB)))
        cases.append((pins_ex.test_ex_leading_dimensions_never_read_padding, dict(transA=tA, transB=tB)))
        cases.append((pins_ex.test_ex_entries_match_full_result_bitwise, dict(transA=tA, transB=tB)))
    cases += [
        (pins_ex.test_ex_beta_zero_never_reads_C, {}),
        (pins_ex.test_ex_alpha_zero_never_reads_A_or_B, {}),
        (pins_ex.test_ex_plain_form_is_the_plain_product, {}),
    ]
    failed = []
    for fn, kw in cases:
        try:
            fn(lib=lib, **kw)
        except AssertionError:
            failed.append(fn.__name__)
    return failed


def test_unmutated_oracle_passes_battery():
    assert _battery(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    assert SOURCE.count(old) == 1, "mutation site not found exactly once"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(SOURCE.replace(old, new))
    out = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(src=str(src), out=out, extra_flags=("-Wno-error",))
    failed = _battery(oracle.load(out))
    assert failed, f"no pin caught mutant {name}"
