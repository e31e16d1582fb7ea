"""Seeded synthetic matrices for the FP32 GEMM tests and benchmark.

This module only draws numbers; it holds none of the product's arithmetic, so
both the HIP path's callers and the CPU oracle's callers can take their inputs
from here without sharing any GEMM code.

Generator: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used counter-style: element i of
a stream with seed s is mix(s + (i + 1) * GAMMA), where GAMMA is the 64-bit
golden-ratio increment and mix() is the published finaliser
(xor-shift 30 / multiply / xor-shift 27 / multiply / xor-shift 31). This is the
same sequence the sequential generator produces from state s, but any element
can be drawn on its own, so a sub-block of a large matrix is reproducible
without generating the rest.

Value maps (all results are exactly representable in float32):

* ``uniform01``  -- the top 24 bits u of each draw, value u * 2**-24, in [0, 1).
* ``uniform_pm1`` -- (u - 2**23) * 2**-23, in [-1, 1).
* ``small_int``  -- integers in [lo, hi] from the top 32 bits (modulo map).
* ``lowp_values`` -- values on the coarser grids that bf16 (8 significant
  bits) or f16 (11) hold exactly, for the reduced-precision workload;
  ``to_lowp_bits`` gives their 16-bit encodings.

The pages draw their inputs from a seeded uniform generator ("Matrix
Multiplication -- Naive to Tiled", section 02: seed 42, rand()/RAND_MAX on
[0, 1]), and time every kernel on identical seeded inputs ("From 306 ms to
86 ms", "How each kernel was timed"). glibc's rand() is not portable, so the
distribution is kept and the generator replaced; the 2**-24 grid keeps every
product of two inputs exact in double precision.
"""

from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Seeds used for the A and B operands of every configuration.
SEED_A = 42
SEED_B = 43


def splitmix64_scalar(seed: int, index: int) -> int:
    """Element ``index`` (0-based) of the SplitMix64 stream seeded with ``seed``,
    in plain Python integers (the definition, used to pin the vector form)."""
    z = (seed + (index + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Elements ``offset .. offset+n-1`` of the stream, as uint64 (wrapping)."""
    with np.errstate(over="ignore"):
        i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
        z = np.uint64(seed & MASK64) + i * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
        return z ^ (z >> np.uint64(31))


def _top24(seed: int, shape) -> np.ndarray:
    n = int(np.prod(shape, dtype=np.int64))
    return (splitmix64(seed, n) >> np.uint64(40)).reshape(shape)


def uniform01(seed: int, shape) -> np.ndarray:
    """float32 matrix with i.i.d. entries u * 2**-24, u uniform on [0, 2**24)."""
    u = _top24(seed, shape).astype(np.float64)
    return (u * 2.0**-24).astype(np.float32)


def uniform_pm1(seed: int, shape) -> np.ndarray:
    """float32 matrix with i.i.d. entries (u - 2**23) * 2**-23 in [-1, 1)."""
    u = _top24(seed, shape).astype(np.int64) - (1 << 23)
    return (u.astype(np.float64) * 2.0**-23).astype(np.float32)


# 16-bit input types of the reduced-precision workload: significant bits of
# the value grid each can hold exactly (bf16: 8, f16: 11, counting the
# implicit bit).
LOWP_BITS = {"bf16": 8, "f16": 11}


def lowp_values(seed: int, shape, dtype: str, dist: str = "u01") -> np.ndarray:
    """float32 matrix of values exactly representable in ``dtype`` ("bf16" or
    "f16"): with b = LOWP_BITS[dtype] and u the top b bits of each draw,
    u * 2**-b in [0, 1) ("u01"), or (u - 2**(b-1)) * 2**-(b-1) in [-1, 1)
    ("pm1"); "int" gives small integers as ``small_int``."""
    if dist == "int":
        return small_int(seed, shape)
    b = LOWP_BITS[dtype]
    n = int(np.prod(shape, dtype=np.int64))
    u = (splitmix64(seed, n) >> np.uint64(64 - b)).reshape(shape).astype(np.int64)
    if dist == "u01":
        return (u.astype(np.float64) * 2.0**-b).astype(np.float32)
    return ((u - (1 << (b - 1))).astype(np.float64) * 2.0**-(b - 1)).astype(np.float32)


def to_lowp_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """The uint16 encodings of float32 values that ``dtype`` holds exactly:
    bf16 is the upper half of the float32 encoding, f16 is IEEE binary16.
    Raises ValueError if a value is not exactly representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32)
        if (u & np.uint32(0xFFFF)).any():
            raise ValueError("value not exactly representable in bf16")
        return (u >> np.uint32(16)).astype(np.uint16)
    if dtype == "f16":
        h = x.astype(np.float16)
        if not np.array_equal(h.astype(np.float32), x, equal_nan=True):
            raise ValueError("value not exactly representable in f16")
        return h.view(np.uint16)
    raise ValueError(f"unknown 16-bit type {dtype!r}")


def small_int(seed: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """float32 matrix of integers in [lo, hi] (top 32 bits modulo the range)."""
    n = int(np.prod(shape, dtype=np.int64))
    t = splitmix64(seed, n) >> np.uint64(32)
    v = (t % np.uint64(hi - lo + 1)).astype(np.int64) + lo
    return v.reshape(shape).astype(np.float32)


def embed(x: np.ndarray, ld: int, fill: float = np.nan) -> np.ndarray:
    """Place a rows x cols matrix in a row-major buffer with leading dimension
    ``ld`` >= cols; the padding columns hold ``fill``. Returns the full
    rows x ld buffer (the logical matrix is ``buf[:, :cols]``)."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    buf = np.full((rows, ld), fill, dtype=np.float32)
    buf[:, :cols] = x
    return buf


# The five workloads: shape (M, N, K), value map, and what they stand for.
WORKLOADS = {
    "sq128": dict(M=128, N=128, K=128, dist="u01"),
    "sq1024": dict(M=1024, N=1024, K=1024, dist="u01"),
    "sq2048": dict(M=2048, N=2048, K=2048, dist="u01"),
    "sq4096": dict(M=4096, N=4096, K=4096, dist="u01"),
    "ragged": dict(M=3001, N=2047, K=4093, dist="pm1"),
}


def operands(M: int, N: int, K: int, dist: str = "u01",
             seed_a: int = SEED_A, seed_b: int = SEED_B):
    """Return (A, B) as contiguous float32 arrays of shape (M, K) and (K, N)."""
    gen = {"u01": uniform01, "pm1": uniform_pm1, "int": small_int}[dist]
    return gen(seed_a, (M, K)), gen(seed_b, (K, N))


# Closed-form integer patterns for products too large to draw on the host: the
# element (r, c) of a pattern (mul_r, mul_c, mod) is ((r * mul_r + c * mul_c)
# mod mod) - mod // 2, a small integer (exact in float32, bf16 and f16 for
# mod <= 33). ``pattern_rows`` gives chosen rows on the host; ``pattern_device``
# fills a whole matrix on a GPU with torch, in row blocks.
def pattern_rows(rows, cols: int, mul_r: int, mul_c: int, mod: int) -> np.ndarray:
    r = np.asarray(rows, dtype=np.int64)[:, None]
    c = np.arange(cols, dtype=np.int64)[None, :]
    return (((r * mul_r + c * mul_c) % mod) - mod // 2).astype(np.float32)


def pattern_device(rows: int, cols: int, mul_r: int, mul_c: int, mod: int, device, dtype=None, block: int = 4096):
    """A rows x cols torch tensor of the pattern on `device` (float32, or
    `dtype`), built a block of rows at a time to bound temporaries."""
    import torch
    out = torch.empty((rows, cols), dtype=dtype or torch.float32, device=device)
    c = torch.arange(cols, dtype=torch.int64, device=device)[None, :] * mul_c
    for r0 in range(0, rows, block):
        r = torch.arange(r0, min(rows, r0 + block), dtype=torch.int64, device=device)[:, None] * mul_r
        out[r0:r0 + r.shape[0]] = (((r + c) % mod) - mod // 2).to(out.dtype)
    return out
