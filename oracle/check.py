"""Acceptance check of a float32 product against the oracle.

TEST INFRASTRUCTURE ONLY.

A float32 result C is accepted when, for every element,

    |C[i][j] - Cref[i][j]| <= REL * S[i][j] + ABS,
    S[i][j] = sum_k |A[i][k]| * |B[k][j]|,

with Cref and S from the oracle in double ("Shared Memory Tiling for Matrix
Multiplication", opening definition of the product, whose terms S sums in
absolute value). Any summation order, FMA contraction or blocking of the
float32 sums is acceptable; the pages only fix the sum itself ("Naive GEMM vs
Tiled GEMM", opening paragraph: tiling leaves the result unchanged). The bound
scales with S, not with |Cref|, because the rounding error of a float32 dot
product is proportional to the sum of the absolute values of its terms, which
cancellation in Cref does not reduce.

The comparison is made as written: the error and the bound are both formed in
double and compared with <=, so an error exactly at the bound passes and the
next double above it fails. NaN or an infinity in C never passes.
"""

from __future__ import annotations

import numpy as np

REL = 1e-5
ABS = 1e-6


def bound(S: np.ndarray) -> np.ndarray:
    """Per-element tolerance REL * S + ABS, in double."""
    return REL * np.asarray(S, dtype=np.float64) + ABS


def error(C: np.ndarray, Cref: np.ndarray) -> np.ndarray:
    """|C - Cref| in double; NaN (from NaN or opposite infinities) becomes inf."""
    err = np.abs(np.asarray(C).astype(np.float64) - np.asarray(Cref, dtype=np.float64))
    return np.where(np.isnan(err), np.inf, err)


def within(C: np.ndarray, Cref: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Boolean array: True where |C - Cref| <= REL * S + ABS."""
    return error(C, Cref) <= bound(S)


def excess(C: np.ndarray, Cref: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Elementwise |C - Cref| / bound, for reporting how close a result came
    to the bound (NaN in C counts as an infinite excess). Acceptance itself is
    decided by ``within``; the two agree, since for doubles x > b > 0 the
    rounded quotient x / b is never 1."""
    return error(C, Cref) / bound(S)


def assert_within(C: np.ndarray, Cref: np.ndarray, S: np.ndarray, what: str = ""):
    """Raise AssertionError naming the worst element if any is out of bound;
    otherwise return the largest error-to-bound ratio."""
    if C.shape != Cref.shape:
        raise AssertionError(f"{what}: shape {C.shape} != {Cref.shape}")
    S = np.broadcast_to(np.asarray(S, dtype=np.float64), C.shape)
    if C.size == 0:
        return 0.0
    ok = within(C, Cref, S)
    r = excess(C, Cref, S)
    if not ok.all():
        bad = ~ok
        idx = tuple(int(i) for i in np.unravel_index(int(np.argmax(np.where(bad, r, -1.0))), r.shape))
        raise AssertionError(
            f"{what}: element {idx} off by {float(error(C[idx], Cref[idx])):.3e} "
            f"(got {float(C[idx])!r}, want {float(Cref[idx])!r}, bound "
            f"{float(bound(S[idx])):.3e}); {int(bad.sum())} of {r.size} out of bound")
    return float(r.max())


def checksum_bound(S_total: float, n_elems: int) -> float:
    """Bound on |sum(C) - sum(Cref)| implied by the elementwise bound: the sum
    over the n_elems elements of REL * S + ABS, i.e. REL * sum(S) + ABS * n."""
    return REL * S_total + ABS * n_elems
