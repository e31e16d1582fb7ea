"""Parity of every kernel variant with the CPU oracle (GPU tests).

Acceptance (per element): |C - Cref| <= 1e-5 * sum_k |A_ik||B_kj| + 1e-6, with
Cref and the sum of absolute products from the oracle in double; bit-exact
where every partial sum is exact (small integers, identity, ones).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import oracle
import synth
from oracle.check import assert_within, checksum_bound
from tests.gpu_util import SENTINEL, gemm

pytestmark = pytest.mark.gpu

VARIANTS = ["naive", "tiled", "regblock", "mfma", "best"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _announce(msg):
    print(f"[parity] {msg}", flush=True)


_REF = {}


def _workload(name):
    """Operands and oracle result of a named workload (cached per module)."""
    if name not in _REF:
        w = synth.WORKLOADS[name]
        A, B = synth.operands(w["M"], w["N"], w["K"], w["dist"])
        if w["dist"] == "u01":       # all terms non-negative: S equals C
            Cref = oracle.gemm(A, B)
            S = Cref
        else:
            Cref, S = oracle.gemm(A, B, with_abs=True)
        _REF[name] = (A, B, Cref, S)
    return _REF[name]


@pytest.mark.parametrize("name", ["sq128", "sq1024", "sq2048", "ragged", "sq4096"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_workloads_elementwise(name, variant):
    _announce(f"workload {name} variant {variant}")
    A, B, Cref, S = _workload(name)
    C = gemm(A, B, variant)
    assert_within(C, Cref, S, f"{name}/{variant}")


TINY = [(m, n, k) for m in (1, 2, 3, 5, 8, 9) for n in (1, 2, 3, 5, 8, 9)
        for k in (1, 2, 3, 5, 8, 9)]


@pytest.mark.parametrize("variant", VARIANTS[:4])
def test_tiny_shapes_brute_force(variant):
    # Tiny shapes: the oracle is exact here (K <= 16), so this is brute force.
    _announce(f"tiny shapes variant {variant}")
    for (M, N, K) in TINY:
        A, B = synth.operands(M, N, K, "pm1", seed_a=M * 100 + K, seed_b=N * 100 + K)
        Cref, S = oracle.gemm(A, B, with_abs=True)
        assert_within(gemm(A, B, variant), Cref, S, f"{variant} {M}x{N}x{K}")


EDGES = [(15, 17, 16), (16, 16, 16), (17, 15, 17), (31, 33, 32), (33, 31, 7),
         (63, 65, 64), (65, 63, 65), (127, 129, 128), (129, 127, 129), (128, 128, 8),
         (255, 257, 256), (257, 255, 33), (256, 256, 255), (1, 300, 129), (300, 1, 129),
         (512, 1024, 768), (130, 258, 1), (200, 136, 24)]


@pytest.mark.parametrize("variant", VARIANTS[:4])
def test_tile_edges(variant):
    _announce(f"tile edges variant {variant}")
    for (M, N, K) in EDGES:
        A, B = synth.operands(M, N, K, "pm1", seed_a=M + 7, seed_b=N + K)
        Cref, S = oracle.gemm(A, B, with_abs=True)
        assert_within(gemm(A, B, variant), Cref, S, f"{variant} {M}x{N}x{K}")


# Aligned shapes that are not whole multiples of the largest tiles: the MFMA
# path then splits the product into whole interior tiles plus bottom and
# right strips (also K tails that are not whole slabs).
SPLIT = [(1000, 1000, 1000), (520, 776, 336), (384, 512, 20), (129, 260, 4100),
         (256, 4, 64), (4, 256, 8), (2048, 1280, 1028)]


@pytest.mark.parametrize("variant", ["mfma", "best"])
def test_interior_and_strip_split(variant):
    _announce(f"interior/strip split variant {variant}")
    for (M, N, K) in SPLIT:
        A, B = synth.operands(M, N, K, "pm1", seed_a=M + 1, seed_b=N + K + 1)
        Cref, S = oracle.gemm(A, B, with_abs=True)
        assert_within(gemm(A, B, variant), Cref, S, f"{variant} {M}x{N}x{K}")
        Ai = synth.small_int(M, (M, K))
        Bi = synth.small_int(N, (K, N))
        assert np.array_equal(gemm(Ai, Bi, variant).astype(np.float64), oracle.gemm(Ai, Bi))


@pytest.mark.parametrize("variant", VARIANTS[:4])
@pytest.mark.parametrize("shape", [(300, 257, 513), (3001, 2047, 4093), (1024, 1024, 1024)])
def test_small_integers_bit_exact(variant, shape):
    # Entries in [-8, 8]: every partial sum is an integer below 2^24, so any
    # summation order gives the exact result.
    M, N, K = shape
    _announce(f"small integers {shape} variant {variant}")
    A = synth.small_int(61, (M, K))
    B = synth.small_int(62, (K, N))
    Cref = oracle.gemm(A, B)
    C = gemm(A, B, variant)
    assert np.array_equal(C.astype(np.float64), Cref)


@pytest.mark.parametrize("variant", VARIANTS[:4])
def test_closed_forms(variant):
    _announce(f"closed forms variant {variant}")
    B = synth.uniform_pm1(71, (200, 130))
    assert np.array_equal(gemm(np.eye(200, dtype=np.float32), B, variant), B)
    A = synth.uniform_pm1(72, (140, 200))
    assert np.array_equal(gemm(A, np.eye(200, dtype=np.float32), variant), A)
    perm = np.random.default_rng(5).permutation(200)
    P = np.zeros((200, 200), np.float32)
    P[np.arange(200), perm] = 1.0
    assert np.array_equal(gemm(P, B, variant), B[perm])
    for K in (1, 37, 4093):
        ones = gemm(np.ones((70, K), np.float32), np.ones((K, 90), np.float32), variant)
        assert np.array_equal(ones, np.full((70, 90), float(K), np.float32))
    d = synth.uniform_pm1(73, (200,))
    assert np.array_equal(gemm(np.diag(d).astype(np.float32), B, variant), d[:, None] * B)


@pytest.mark.parametrize("variant", VARIANTS[:4])
def test_strided_views_and_misaligned_starts(variant):
    # Sub-matrices of larger buffers (NaN in the padding of A and B, a
    # sentinel around C): the result must equal the packed run bit for bit,
    # and nothing outside C's window may change.
    M, N, K = 150, 260, 333
    _announce(f"strided views variant {variant}")
    A, B = synth.operands(M, N, K, "pm1", seed_a=81, seed_b=82)
    packed = gemm(A, B, variant)
    for pads, offs in [((4, 4, 4), (0, 0, 0)), ((3, 5, 7), (0, 0, 0)),
                       ((0, 0, 0), (1, 2, 3)), ((5, 1, 9), (3, 1, 2))]:
        C, cbuf, ldc, off = gemm(A, B, variant, ld_pad=pads, offset=offs, return_buffer=True)
        assert np.array_equal(C, packed), (pads, offs)
        mask = np.ones(cbuf.shape, bool)
        idx = off + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        mask[idx.ravel()] = False
        assert (cbuf[mask] == SENTINEL).all(), (pads, offs)


@pytest.mark.parametrize("variant", VARIANTS[:4])
def test_overwrites_and_empty_sum(variant):
    _announce(f"overwrite / K=0 variant {variant}")
    # C starts as SENTINEL in gemm(); a K = 0 product must be all zeros.
    z = gemm(np.zeros((70, 0), np.float32), np.zeros((0, 130), np.float32), variant)
    assert np.array_equal(z, np.zeros((70, 130), np.float32))
    A, B = synth.operands(65, 67, 5, "u01")
    C = gemm(A, B, variant)
    assert np.isfinite(C).all() and (C != SENTINEL).all()


@pytest.mark.parametrize("variant", VARIANTS[:4])
def test_repeat_runs_identical(variant):
    # No atomics and no split reduction: identical bytes on every run (a race
    # on LDS would show up as run-to-run differences).
    _announce(f"determinism variant {variant}")
    A, B = synth.operands(1000, 1100, 1300, "pm1", seed_a=91, seed_b=92)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    first = sg.matmul(dA, dB, variant=variant).cpu()
    for _ in range(4):
        assert torch.equal(sg.matmul(dA, dB, variant=variant).cpu(), first)


def test_side_stream_and_matmul_api():
    A, B = synth.operands(300, 200, 100, "pm1", seed_a=3, seed_b=4)
    Cref, S = oracle.gemm(A, B, with_abs=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = sg.matmul(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda())
    s.synchronize()
    assert_within(C.cpu().numpy(), Cref, S, "side stream")
    # matmul on views of larger tensors
    big = torch.from_numpy(synth.uniform_pm1(5, (400, 300))).cuda()
    a, b = big[:300, :100], big[100:200, 50:250]
    Cref2, S2 = oracle.gemm(a.cpu().numpy(), b.cpu().numpy(), with_abs=True)
    assert_within(sg.matmul(a, b).cpu().numpy(), Cref2, S2, "views")


def test_headline_checksum_and_freivalds():
    # Whole-matrix properties of the 4096^3 product as the benchmark runs it:
    # the check sum (exact in integers via column sums of A and row sums of B)
    # and a Freivalds probe C x = A (B x) for random signs x.
    _announce("headline checksum / Freivalds")
    A, B, Cref, S = _workload("sq4096")
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = sg.matmul(dA, dB, variant="best")
    torch.cuda.synchronize()
    Cn = C.cpu().numpy()
    ia = (A.astype(np.float64) * 2**24).astype(np.int64)
    ib = (B.astype(np.float64) * 2**24).astype(np.int64)
    exact = Fraction(sum(int(x) * int(y) for x, y in
                         zip(ia.sum(axis=0).tolist(), ib.sum(axis=1).tolist())), 2**48)
    got = Fraction(math.fsum(Cn.astype(np.float64).ravel().tolist()))
    bound = checksum_bound(float(exact), Cn.size)      # S == C for these inputs
    assert abs(float(got - exact)) <= bound
    x = np.random.default_rng(11).choice([-1.0, 1.0], size=4096)
    lhs = Cn.astype(np.float64) @ x
    rhs = A.astype(np.float64) @ (B.astype(np.float64) @ x)
    row_bound = 1e-5 * S.sum(axis=1) + 1e-6 * 4096 + 1e-9 * np.abs(Cref).sum(axis=1)
    assert (np.abs(lhs - rhs) <= row_bound).all()
