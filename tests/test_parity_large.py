"""Products past 2^31 elements (GPU tests): the maximum-size cases.

Offsets are formed in 64 bits everywhere; these tests make them matter. One
operand (A, stored either way) holds more than 2^31 elements, or C does, for
every kernel variant, the split schedule and the 16-bit kernels. The inputs
are closed-form small-integer patterns (synth.pattern_device fills them on the
GPU; synth.pattern_rows gives the sampled rows on the host), so every sum is
exact and the sampled elements must equal the oracle's bit for bit: rows on
both sides of the 2^31-element mark, the last rows and the last columns.
"""

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import oracle
import synth

pytestmark = pytest.mark.gpu

A_PAT = (7, 13, 17)   # op(A)[r][k] = ((7 r + 13 k) mod 17) - 8
B_PAT = (5, 3, 11)    # op(B)[k][c] = ((5 k + 3 c) mod 11) - 5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _op_a_device(M, K, trans, dtype=None):
    """op(A) = pattern (M x K), stored M x K, or K x M when trans."""
    mr, mc, mod = A_PAT
    if trans:
        return synth.pattern_device(K, M, mc, mr, mod, "cuda", dtype)
    return synth.pattern_device(M, K, mr, mc, mod, "cuda", dtype)


def _expected(rows, cols, K):
    """Oracle values at (rows[e], cols[e]) of op(A) op(B), from the sampled rows of op(A)."""
    uniq, inv = np.unique(rows, return_inverse=True)
    A_sub = synth.pattern_rows(uniq, K, *A_PAT)
    B = synth.pattern_rows(np.arange(K), int(cols.max()) + 1, *B_PAT)
    want, _ = oracle.gemm_entries(A_sub, B, inv, cols)
    return want


def _samples(M, N, mark_row, rng):
    rows = np.concatenate([rng.integers(0, M, 200), np.arange(mark_row - 8, mark_row + 8), np.arange(M - 8, M)])
    rows = rows[(rows >= 0) & (rows < M)]
    cols = np.concatenate([rng.integers(0, N, rows.size - 16), np.full(16, N - 1)])
    return rows, cols


M1, K1, N1 = 65600, 32768, 72      # op(A): 2.15e9 elements


@pytest.mark.parametrize("variant", ["naive", "tiled", "regblock", "mfma"])
@pytest.mark.parametrize("trans_a", [False, True], ids=["a", "at"])
def test_operand_past_2_31_elements(trans_a, variant):
    print(f"[large] A {M1}x{K1} trans={trans_a} {variant}", flush=True)
    dA = _op_a_device(M1, K1, trans_a)
    dB = synth.pattern_device(K1, N1, *B_PAT, "cuda")
    dC = torch.full((M1, N1), float("nan"), device="cuda")
    ta = sg.SGEMM_OP_T if trans_a else sg.SGEMM_OP_N
    rc = sg.sgemm_ex(ta, sg.SGEMM_OP_N, M1, N1, K1, 1.0, dA.data_ptr(), M1 if trans_a else K1, dB.data_ptr(), N1,
                     0.0, dC.data_ptr(), N1, torch.cuda.current_stream().cuda_stream, sg.VARIANTS[variant])
    assert rc == sg.SGEMM_OK
    torch.cuda.synchronize()
    rows, cols = _samples(M1, N1, (1 << 31) // K1, np.random.default_rng(1))
    got = dC.cpu().numpy()[rows, cols]
    assert np.array_equal(got.astype(np.float64), _expected(rows, cols, K1))


def test_split_schedule_past_2_31_elements():
    need = sg.sgemm_ex_workspace_size(sg.SGEMM_OP_N, sg.SGEMM_OP_N, M1, N1, K1,
                                      torch.cuda.get_device_properties(0).multi_processor_count)
    if need == 0:
        pytest.skip("the library keeps this product on whole tiles")
    print(f"[large] split schedule, workspace {need >> 20} MiB", flush=True)
    dA = _op_a_device(M1, K1, False)
    dB = synth.pattern_device(K1, N1, *B_PAT, "cuda")
    dC = torch.full((M1, N1), float("nan"), device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = sg.sgemm_ex_ws(sg.SGEMM_OP_N, sg.SGEMM_OP_N, M1, N1, K1, 1.0, dA.data_ptr(), K1, dB.data_ptr(), N1, 0.0,
                        dC.data_ptr(), N1, ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream,
                        sg.SGEMM_MFMA)
    assert rc == sg.SGEMM_OK
    torch.cuda.synchronize()
    rows, cols = _samples(M1, N1, (1 << 31) // K1, np.random.default_rng(2))
    got = dC.cpu().numpy()[rows, cols]
    assert np.array_equal(got.astype(np.float64), _expected(rows, cols, K1))


@pytest.mark.parametrize("trans_a", [False, True], ids=["a", "at"])
def test_lowp_operand_past_2_31_elements(trans_a):
    print(f"[large] bf16 A {M1}x{K1} trans={trans_a}", flush=True)
    dA = _op_a_device(M1, K1, trans_a, torch.bfloat16)
    dB = synth.pattern_device(K1, N1, *B_PAT, "cuda", torch.bfloat16)
    dC = torch.full((M1, N1), float("nan"), device="cuda")
    ta = sg.SGEMM_OP_T if trans_a else sg.SGEMM_OP_N
    rc = sg.sgemm_lp(sg.SGEMM_LP_BF16, ta, sg.SGEMM_OP_N, M1, N1, K1, 1.0, dA.data_ptr(), M1 if trans_a else K1,
                     dB.data_ptr(), N1, 0.0, dC.data_ptr(), N1, torch.cuda.current_stream().cuda_stream)
    assert rc == sg.SGEMM_OK
    torch.cuda.synchronize()
    rows, cols = _samples(M1, N1, (1 << 31) // K1, np.random.default_rng(3))
    got = dC.cpu().numpy()[rows, cols]
    assert np.array_equal(got.astype(np.float64), _expected(rows, cols, K1))


M2 = N2 = 46400   # C: 2.15e9 elements
K2 = 24


@pytest.mark.parametrize("variant", ["naive", "tiled", "regblock", "mfma"])
def test_output_past_2_31_elements(variant):
    print(f"[large] C {M2}x{N2} {variant}", flush=True)
    dA = _op_a_device(M2, K2, False)
    dB = synth.pattern_device(K2, N2, *B_PAT, "cuda")
    dC = torch.full((M2, N2), float("nan"), device="cuda")
    rc = sg.sgemm(M2, N2, K2, dA.data_ptr(), K2, dB.data_ptr(), N2, dC.data_ptr(), N2,
                  torch.cuda.current_stream().cuda_stream, sg.VARIANTS[variant])
    assert rc == sg.SGEMM_OK
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    mark = (1 << 31) // N2
    rows = np.concatenate([rng.integers(0, M2, 300), np.arange(mark - 4, mark + 4), np.full(8, M2 - 1)])
    cols = np.concatenate([rng.integers(0, N2, 300), rng.integers(0, N2, 8), np.arange(N2 - 8, N2)])
    got = dC[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    assert np.array_equal(got.astype(np.float64), _expected(rows, cols, K2))
    assert not torch.isnan(dC).any().item()          # every element written
