"""The split ("stream-K") schedule of sgemm_ex_ws (GPU tests).

Products whose tiles would load the compute units unevenly are dealt out by
(tile, K slab) iteration to one work-group per compute unit; tiles shared by
several work-groups go through the workspace and are added in K order by a
second kernel. These tests run products the library puts on that schedule
(checked on the host with sgemm_ex_workspace_size), with every transpose
pair, alpha and beta, ragged edges and a partial last K slab, against the
oracle; and check that results repeat bit for bit, that the workspace's prior
contents do not matter, that nothing outside C's window is written, and that
a missing, short or misaligned workspace gives exactly sgemm_ex.
"""

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import oracle
import synth
from oracle.check import assert_within
from tests.gpu_util import SENTINEL, gemm_ex

pytestmark = pytest.mark.gpu

PAIRS = [(False, False), (False, True), (True, False), (True, True)]
PAIR_IDS = ["nn", "nt", "tn", "tt"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


@pytest.fixture(scope="module")
def workspace():
    return torch.full((160 << 20,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-like junk


def _stored(x, trans):
    return np.ascontiguousarray(x.T) if trans else x


def _split_bytes(tA, tB, M, N, K):
    return sg.sgemm_ex_workspace_size(int(tA), int(tB), M, N, K, torch.cuda.get_device_properties(0).multi_processor_count)


def _sampled_check(tA, tB, alpha, A, B, beta, C0, C, what):
    M, N = C0.shape
    rng = np.random.default_rng(M * 7 + N)
    rows = np.concatenate([rng.integers(0, M, 3000), np.arange(max(0, M - 40), M).repeat(8)])
    cols = np.concatenate([rng.integers(0, N, 3000), np.arange(max(0, N - 40), N).repeat(8)])
    rows, cols = rows[: min(rows.size, cols.size)], cols[: min(rows.size, cols.size)]
    want, S = oracle.gemm_ex_entries(tA, tB, alpha, A, B, beta, C0, rows, cols)
    assert_within(C[rows, cols], want, S, what)


# (M, N, K): ragged edges with a K tail, an exact fit, a deep-K thin product
# and a square one, all put on the split schedule by the library.
SHAPES = [(2047, 2560, 4093), (2560, 2560, 2560), (1000, 1000, 8000), (3072, 3072, 3072), (517, 509, 16001)]


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_split_schedule_matches_oracle(shape, pair, workspace):
    M, N, K = shape
    tA, tB = pair
    need = _split_bytes(tA, tB, M, N, K)
    assert 0 < need <= workspace.numel(), (shape, need)
    print(f"[split] {M}x{N}x{K} {pair} workspace {need >> 20} MiB", flush=True)
    opA = synth.uniform_pm1(M + 1, (M, K))
    opB = synth.uniform_pm1(N + 2, (K, N))
    C0 = synth.uniform_pm1(K + 3, (M, N))
    A, B = _stored(opA, tA), _stored(opB, tB)
    C = gemm_ex(tA, tB, -0.75, A, B, 1.25, C0, "mfma", workspace=workspace)
    _sampled_check(tA, tB, -0.75, A, B, 1.25, C0, C, f"split {shape} {pair}")


def test_split_schedule_small_integers_bit_exact(workspace):
    # Every partial sum is an integer below 2^24: exact in any order, so the
    # split sums equal the float64 product bit for bit.
    M, N, K = 1000, 1000, 8000
    print("[split] small integers", flush=True)
    A = synth.small_int(5, (M, K), -4, 4)
    B = synth.small_int(6, (K, N), -4, 4)
    assert _split_bytes(False, False, M, N, K) > 0
    C = gemm_ex(False, False, 1.0, A, B, 0.0, np.zeros((M, N), np.float32), "mfma", workspace=workspace)
    assert np.array_equal(C.astype(np.float64), A.astype(np.float64) @ B.astype(np.float64))


def test_split_schedule_repeats_and_ignores_workspace_contents(workspace):
    M, N, K = 2047, 2560, 4093
    print("[split] repeatability", flush=True)
    A = synth.uniform_pm1(11, (M, K))
    B = synth.uniform_pm1(12, (K, N))
    C0 = np.zeros((M, N), np.float32)
    C1 = gemm_ex(False, False, 1.0, A, B, 0.0, C0, "best", workspace=workspace)
    workspace.fill_(0x7F)
    C2 = gemm_ex(False, False, 1.0, A, B, 0.0, C0, "best", workspace=workspace)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


def test_split_schedule_writes_only_the_window(workspace):
    M, N, K = 2047, 2560, 4093
    print("[split] window", flush=True)
    A = synth.uniform_pm1(21, (M, K))
    B = synth.uniform_pm1(22, (K, N))
    C0 = synth.uniform_pm1(23, (M, N))
    C, buf, ldc, off = gemm_ex(False, False, 0.5, A, B, -1.0, C0, "mfma", ld_pad=(3, 5, 7), offset=(1, 2, 3),
                               return_buffer=True, workspace=workspace)
    inside = np.zeros(buf.shape, bool)
    for r in range(M):
        inside[off + r * ldc: off + r * ldc + N] = True
    assert (buf[~inside] == SENTINEL).all()
    _sampled_check(False, False, 0.5, A, B, -1.0, C0, C, "split, padded")


def test_short_or_missing_workspace_is_exactly_sgemm_ex(workspace):
    M, N, K = 2560, 2560, 2560
    print("[split] fallback", flush=True)
    need = _split_bytes(False, True, M, N, K)
    assert need > 0
    A = synth.uniform_pm1(31, (M, K))
    B = np.ascontiguousarray(synth.uniform_pm1(32, (K, N)).T)
    C0 = synth.uniform_pm1(33, (M, N))
    plain = gemm_ex(False, True, 2.0, A, B, 0.5, C0, "mfma")
    short = gemm_ex(False, True, 2.0, A, B, 0.5, C0, "mfma", workspace=workspace[: need - 1])
    empty = gemm_ex(False, True, 2.0, A, B, 0.5, C0, "mfma", workspace=workspace[:0])
    # Large enough but not 16-byte aligned (the fixture's storage is).
    assert workspace.data_ptr() % 16 == 0
    skewed = gemm_ex(False, True, 2.0, A, B, 0.5, C0, "mfma", workspace=workspace[4:4 + need])
    assert np.array_equal(plain.view(np.uint32), short.view(np.uint32))
    assert np.array_equal(plain.view(np.uint32), empty.view(np.uint32))
    assert np.array_equal(plain.view(np.uint32), skewed.view(np.uint32))
    # Other variants ignore the workspace.
    tiled = gemm_ex(False, True, 2.0, A, B, 0.5, C0, "tiled")
    tiled_ws = gemm_ex(False, True, 2.0, A, B, 0.5, C0, "tiled", workspace=workspace)
    assert np.array_equal(tiled.view(np.uint32), tiled_ws.view(np.uint32))


def test_products_left_on_whole_tiles_are_unchanged(workspace):
    # Where the model keeps whole tiles (here 2048^3, 4096 x 4096 x 256 and
    # 3001 x 2047 x 4093, one 192 x 128 tile per compute unit), sgemm_ex_ws is
    # sgemm_ex bit for bit.
    print("[split] whole-tile products", flush=True)
    for (M, N, K) in [(2048, 2048, 2048), (4096, 4096, 256), (3001, 2047, 4093)]:
        assert _split_bytes(False, False, M, N, K) == 0
        A = synth.uniform_pm1(41, (M, K))
        B = synth.uniform_pm1(42, (K, N))
        C0 = np.zeros((M, N), np.float32)
        a = gemm_ex(False, False, 1.0, A, B, 0.0, C0, "mfma")
        b = gemm_ex(False, False, 1.0, A, B, 0.0, C0, "mfma", workspace=workspace)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_tensor_api_workspace(workspace):
    print("[split] tensor api", flush=True)
    M, N, K = 1536, 1536, 1536
    A = torch.from_numpy(synth.uniform_pm1(51, (M, K))).cuda()
    B = torch.from_numpy(synth.uniform_pm1(52, (N, K))).cuda().t()   # a transposed view
    C = sg.gemm(A, B, workspace=workspace)
    torch.cuda.synchronize()
    Cref, S = oracle.gemm_ex(False, True, 1.0, A.cpu().numpy(), B.t().contiguous().cpu().numpy(), 0.0,
                             np.zeros((M, N), np.float32))
    assert_within(C.cpu().numpy(), Cref, S, "tensor api with workspace")
    with pytest.raises(ValueError):
        sg.gemm(A, B, workspace=workspace.cpu()[:16])
