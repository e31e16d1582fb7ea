"""Acceptance check of a float32 product against the oracle.

TEST INFRASTRUCTURE ONLY.

A float32 result C is accepted when, for every element,

    |C[i][j] - Cref[i][j]| <= REL * S[i][j] + ABS,
    S[i][j] = sum_k |A[i][k]| * |B[k][j]|,

with Cref and S from the oracle in double. Any summation order, FMA
contraction or blocking of the float32 sums is acceptable; the pages only fix
the sum itself ("Naive GEMM vs Tiled GEMM", opening paragraph: tiling gives the
same answer). The bound scales with S because the rounding error of a float32
dot product is proportional to the sum of the absolute values of its terms.
"""

from __future__ import annotations

import numpy as np

REL = 1e-5
ABS = 1e-6


def bound(S: np.ndarray) -> np.ndarray:
    return REL * S + ABS


def excess(C: np.ndarray, Cref: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Elementwise |C - Cref| / bound; accepted iff every value is <= 1.
    NaN in C counts as an infinite excess."""
    err = np.abs(C.astype(np.float64) - Cref)
    err = np.where(np.isnan(err), np.inf, err)
    return err / bound(S)


def assert_within(C: np.ndarray, Cref: np.ndarray, S: np.ndarray, what: str = ""):
    """Raise AssertionError naming the worst element if any is out of bound."""
    if C.shape != Cref.shape:
        raise AssertionError(f"{what}: shape {C.shape} != {Cref.shape}")
    if C.size == 0:
        return 0.0
    r = excess(C, Cref, S)
    worst = float(r.max())
    if not worst <= 1.0:
        idx = np.unravel_index(int(np.argmax(r)), r.shape)
        raise AssertionError(
            f"{what}: element {idx} off by {abs(float(C[idx]) - Cref[idx]):.3e} "
            f"(got {float(C[idx])!r}, want {Cref[idx]!r}, bound "
            f"{bound(S[idx]):.3e}); {int((r > 1).sum())} of {r.size} out of bound")
    return worst


def checksum_bound(S_total: float, n_elems: int) -> float:
    """Bound on |sum(C) - sum(Cref)| implied by the elementwise bound:
    the sum of the elementwise bounds."""
    return REL * S_total + ABS * n_elems
