"""The operation count behind the benchmark's rate, pinned to the pages' own
worked figures (tests/golden/flop_rates.txt, each row citing its page).

"Matrix Multiplication -- Naive to Tiled" (sections 03 and 06) and "Naive
GEMM vs Tiled GEMM" print total FLOP counts and times with the rates they give.
bench.flops() must reproduce every printed rate from its printed time, within
the interval the printed rounding of both numbers leaves. A count off by a
factor (M*N*K without the 2, or an extra K) fails every row.
"""

import math
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "flop_rates.txt")
UNIT = {"FLOP": 1.0, "GFLOPS": 1e9, "TFLOP/s": 1e12}


def _rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kind, mnk, ms, value, unit, source = [f.strip() for f in line.split("|", 5)]
        M, N, K = (int(x) for x in mnk.split())
        rows.append((kind, M, N, K, ms, value, unit, source))
    return rows


def _half_ulp(printed: str) -> float:
    """Half a unit in the last printed place ("0.12" -> 0.005, "2.15e9" ->
    0.005e9, "1217" -> 0.5)."""
    mant, _, exp = printed.lower().partition("e")
    decimals = len(mant.split(".")[1]) if "." in mant else 0
    return 0.5 * 10.0 ** (-decimals) * 10.0 ** (int(exp) if exp else 0)


ROWS = _rows()


def test_fixture_has_every_kind():
    kinds = [r[0] for r in ROWS]
    assert kinds.count("flop") >= 1 and kinds.count("rate") >= 12 and kinds.count("inconsistent") >= 1


@pytest.mark.parametrize("row", [r for r in ROWS if r[0] == "flop"], ids=lambda r: f"{r[1]}^3")
def test_printed_flop_count(row):
    _, M, N, K, _, value, unit, source = row
    got = bench.flops(M, N, K) / UNIT[unit]
    assert abs(got - float(value)) <= _half_ulp(value), (source, got)


@pytest.mark.parametrize("row", [r for r in ROWS if r[0] == "rate"], ids=lambda r: f"{r[1]}^3-{r[4]}ms")
def test_printed_rate_follows_from_printed_time(row):
    _, M, N, K, ms, value, unit, source = row
    f = bench.flops(M, N, K) / UNIT[unit]
    t, dt = float(ms) * 1e-3, _half_ulp(ms) * 1e-3
    lo, hi = f / (t + dt), f / (t - dt)          # rates the rounded time allows
    v, dv = float(value), _half_ulp(value)
    assert lo <= v + dv and v - dv <= hi, (source, lo, hi, v)


@pytest.mark.parametrize("row", [r for r in ROWS if r[0] == "inconsistent"], ids=lambda r: f"{r[1]}^3")
def test_inconsistent_row_really_is(row):
    # Kept in the fixture to document the reading: the printed pair cannot both
    # hold at the size the page's table uses.
    _, M, N, K, ms, value, unit, source = row
    got = bench.flops(M, N, K) / UNIT[unit] / (float(ms) * 1e-3)
    assert not math.isclose(got, float(value), rel_tol=0.1), (source, got)


def test_a_wrong_count_fails_the_rates():
    # The pins above must reject plausible mistakes in the count.
    for wrong in (lambda M, N, K: M * N * K, lambda M, N, K: 4 * M * N * K, lambda M, N, K: 2 * M * N):
        bad = 0
        for kind, M, N, K, ms, value, unit, _ in ROWS:
            if kind != "rate":
                continue
            f = wrong(M, N, K) / UNIT[unit]
            t, dt = float(ms) * 1e-3, _half_ulp(ms) * 1e-3
            v, dv = float(value), _half_ulp(value)
            if not (f / (t + dt) <= v + dv and v - dv <= f / (t - dt)):
                bad += 1
        assert bad >= 10
