"""Pins of the acceptance check (host only).

Every GPU parity test and the bench's sampled check decide pass or fail
through ``oracle/check.py``: an element passes when
|C - Cref| <= 1e-5 * S + 1e-6, with S = sum_k |A_ik| |B_kj| ("Shared Memory
Tiling for Matrix Multiplication", opening definition of the product; the
bound is the library's stated tolerance). These tests fix that rule on
hand-built C, Cref and S, where the right answer is known without the check:
values exactly at the bound and one double past it, results whose error lies
between REL * |Cref| and REL * S (they differ once signs cancel), NaN and
infinities, one bad element among a million, and the checksum bound's two
terms. ``test_planted_mistake_is_caught`` then plants plausible mistakes in
copies of the check and requires each to fail at least one of these cases.
"""

import importlib.util

import numpy as np
import pytest

import oracle.check as check_module

REL = 1e-5
ABS = 1e-6


def _at_bound_values(rng, n=4096):
    """S values spread over many binades (including 0), and the double
    bound b = REL * S + ABS of each, formed exactly as the rule states."""
    S = np.concatenate([[0.0, 1.0, 1e-6, 0.5, 4096.0, 1.7e7],
                        10.0 ** rng.uniform(-8, 8, n - 6)])
    return S, REL * S + ABS


def case_error_exactly_at_bound_passes(chk, rng):
    S, b = _at_bound_values(rng)
    C = np.zeros(S.shape, np.float32)
    # C - Cref is exactly -b or +b: both signs sit on the bound and pass.
    chk.assert_within(C, b.copy(), S, "at bound, C below")
    chk.assert_within(C, -b, S, "at bound, C above")
    assert chk.within(C, b, S).all()


def case_next_double_past_bound_fails(chk, rng):
    S, b = _at_bound_values(rng)
    C = np.zeros(S.shape, np.float32)
    past = np.nextafter(b, np.inf)
    # Every element fails on its own: check one element at a time.
    for i in range(S.size):
        with pytest.raises(AssertionError):
            chk.assert_within(C[i:i + 1], past[i:i + 1], S[i:i + 1], "past bound")
        with pytest.raises(AssertionError):
            chk.assert_within(C[i:i + 1], -past[i:i + 1], S[i:i + 1], "past bound")
    assert not chk.within(C, past, S).any()


def case_bound_uses_S_not_Cref(chk, rng):
    # Hand-built: Cref = 0.01, S = 1000, so REL*S + ABS = 0.010001 but
    # REL*|Cref| + ABS = 1.01e-6. An error of 0.01 passes only on S.
    C = np.zeros(3, np.float32)
    Cref = np.array([0.01, -0.01, 0.0078125])
    S = np.array([1000.0, 1000.0, 1000.0])
    chk.assert_within(C, Cref, S, "error below REL*S, above REL*|Cref|")
    # And just past REL*S + ABS it fails, whatever |Cref| is.
    with pytest.raises(AssertionError):
        chk.assert_within(C[:1], np.array([0.0100011]), S[:1], "past REL*S")
    # A product of U[-1,1) operands: signs cancel, so S is several times
    # |Cref|. Half the allowed error on every element must pass.
    A = rng.integers(-2**23, 2**23, (64, 64)) * 2.0**-23
    B = rng.integers(-2**23, 2**23, (64, 64)) * 2.0**-23
    Cref = A @ B
    Sv = np.abs(A) @ np.abs(B)
    assert (Sv > 3 * np.abs(Cref)).mean() > 0.5
    C = (Cref + 0.5 * REL * Sv).astype(np.float32)
    chk.assert_within(C, Cref, Sv, "half the bound, signed inputs")
    assert not chk.within((Cref + 1.5 * REL * Sv + ABS).astype(np.float32), Cref, Sv).any()


def case_error_of_either_sign_counts(chk, rng):
    S, b = _at_bound_values(rng, 256)
    C = np.zeros(S.shape, np.float32)
    for sign in (1.0, -1.0):
        with pytest.raises(AssertionError):
            chk.assert_within(C, sign * 2.0 * b, S, "twice the bound")


def case_nan_and_infinities_never_pass(chk, rng):
    Cref = np.full(8, 3.0)
    S = np.full(8, 1e30)          # a bound so loose that any finite C passes
    for bad in (np.nan, np.inf, -np.inf):
        C = np.full(8, 3.0, np.float32)
        C[5] = bad
        with pytest.raises(AssertionError):
            chk.assert_within(C, Cref, S, f"C holds {bad}")
        assert not chk.within(C, Cref, S)[5]
        assert np.isinf(chk.excess(C, Cref, S)[5])


def case_one_bad_element_among_a_million(chk, rng):
    Cref = rng.integers(0, 2**20, (1000, 1000)).astype(np.float64)
    S = np.abs(Cref)
    C = Cref.astype(np.float32)
    assert chk.assert_within(C, Cref, S, "exact") == 0.0
    C[617, 401] += np.float32(64.0)
    with pytest.raises(AssertionError, match=r"\(617, 401\)"):
        chk.assert_within(C, Cref, S, "one bad element")


def case_difference_taken_in_double(chk, rng):
    # Cref = 2^24 + 0.9 rounds to C = 2^24 in float32; the error is 0.9,
    # far past the bound ABS of S = 0. A float32 subtraction would see 0.
    C = np.array([2.0**24], np.float32)
    with pytest.raises(AssertionError):
        chk.assert_within(C, np.array([2.0**24 + 0.9]), np.array([0.0]), "float32 diff")


def case_returns_worst_ratio(chk, rng):
    Cref = np.array([1.0, 2.0, 4.0])
    S = np.array([1e5, 1e5, 1e5])          # bound = 1.000001
    C = np.array([1.5, 2.0, 4.25], np.float32)
    r = chk.assert_within(C, Cref, S, "ratios")
    assert r == pytest.approx(0.5 / (REL * 1e5 + ABS), rel=1e-15)


def case_shapes_must_match(chk, rng):
    with pytest.raises(AssertionError):
        chk.assert_within(np.zeros((3, 4), np.float32), np.zeros((4, 3)),
                          np.zeros((4, 3)), "transposed")
    assert chk.assert_within(np.zeros((0, 5), np.float32), np.zeros((0, 5)),
                             np.zeros((0, 5)), "empty") == 0.0


def case_checksum_bound_is_the_sum_of_elementwise_bounds(chk, rng):
    assert chk.checksum_bound(0.0, 10**6) == pytest.approx(1.0, rel=1e-15)
    assert chk.checksum_bound(1e6, 0) == pytest.approx(10.0, rel=1e-15)
    S = rng.uniform(0, 4096, (300, 200))
    assert chk.checksum_bound(float(S.sum()), S.size) == pytest.approx(
        float((REL * S + ABS).sum()), rel=1e-12)


CASES = [v for k, v in sorted(globals().items()) if k.startswith("case_")]


@pytest.mark.parametrize("case", CASES, ids=[c.__name__[5:] for c in CASES])
def test_check(case):
    case(check_module, np.random.default_rng(2024))


with open(check_module.__file__) as f:
    SOURCE = f.read()

# Plausible mistakes in the check, one site each.
MUTANTS = {
    "drops_abs": ("err = np.abs(np.asarray(C).astype(np.float64) - np.asarray(Cref, dtype=np.float64))",
                  "err = np.asarray(C).astype(np.float64) - np.asarray(Cref, dtype=np.float64)"),
    "bound_from_abs_Cref": ("ok = within(C, Cref, S)", "ok = within(C, Cref, np.abs(Cref))"),
    "within_bound_from_abs_Cref": ("return error(C, Cref) <= bound(S)",
                                   "return error(C, Cref) <= bound(np.abs(Cref))"),
    "strict_less_than": ("return error(C, Cref) <= bound(S)", "return error(C, Cref) < bound(S)"),
    "nan_counts_as_zero": ("return np.where(np.isnan(err), np.inf, err)",
                           "return np.where(np.isnan(err), 0.0, err)"),
    "any_instead_of_all": ("if not ok.all():", "if not ok.any():"),
    "bound_drops_abs_term": ("return REL * np.asarray(S, dtype=np.float64) + ABS",
                             "return REL * np.asarray(S, dtype=np.float64)"),
    "bound_sqrt_S": ("return REL * np.asarray(S, dtype=np.float64) + ABS",
                     "return REL * np.sqrt(np.asarray(S, dtype=np.float64)) + ABS"),
    "float32_difference": ("np.asarray(C).astype(np.float64) - np.asarray(Cref, dtype=np.float64)",
                           "(np.asarray(C, dtype=np.float32) - np.asarray(Cref).astype(np.float32)).astype(np.float64)"),
    "checksum_drops_abs_term": ("return REL * S_total + ABS * n_elems", "return REL * S_total"),
    "checksum_drops_rel_term": ("return REL * S_total + ABS * n_elems", "return ABS * n_elems"),
    "shape_unchecked": ("if C.shape != Cref.shape:", "if C.ndim != Cref.ndim:"),
}


def _load(path, name):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _battery(chk):
    failed = []
    for case in CASES:
        try:
            case(chk, np.random.default_rng(2024))
        except (Exception, pytest.fail.Exception):  # a mutant may fail in any way
            failed.append(case.__name__)
    return failed


def test_unmutated_check_passes_battery(tmp_path):
    path = tmp_path / "check_copy.py"
    path.write_text(SOURCE)
    assert _battery(_load(str(path), "check_copy")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SOURCE.count(old) == 1, "mutation site not found exactly once"
    path = tmp_path / f"check_{name}.py"
    path.write_text(SOURCE.replace(old, new))
    failed = _battery(_load(str(path), f"check_{name}"))
    assert failed, f"no case caught mutant {name}"
