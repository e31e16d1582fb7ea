"""sgemm_ex_noalloc against sgemm_ex_ws (GPU tests, through the C ABI).

sgemm_ex_noalloc is sgemm_ex_ws with the split schedule's partial tiles in
the library's own static device buffer instead of a caller's workspace, for
callers that cannot allocate. On the same product it runs the same kernels
on the same plan, so its C must equal sgemm_ex_ws's bit for bit (and lie
within the acceptance bound of the oracle, exact on small integers). Calls in
a row share the buffer: the second call here is smaller than the first, so
it runs over what the first left behind.
"""

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import oracle
import synth
from oracle.check import assert_within

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run(entry, M, N, K, A, B, C0, alpha, beta, ws=None, tA=False, tB=False):
    """One call of sgemm_ex_noalloc ("noalloc") or sgemm_ex_ws ("ws") on
    device copies; returns C."""
    dA, dB, dC = _dev(A), _dev(B), _dev(C0)
    s = torch.cuda.current_stream()
    lda, ldb = A.shape[1], B.shape[1]
    ta, tb = int(tA), int(tB)
    if entry == "noalloc":
        rc = sg.sgemm_ex_noalloc(ta, tb, M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta,
                                 dC.data_ptr(), N, s.cuda_stream, sg.SGEMM_BEST)
    else:
        rc = sg.sgemm_ex_ws(ta, tb, M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta, dC.data_ptr(), N,
                            ws.data_ptr(), ws.numel(), s.cuda_stream, sg.SGEMM_BEST)
    assert rc == sg.SGEMM_OK, sg.sgemm_status_string(rc)
    s.synchronize()
    return dC.cpu().numpy()


# Two calls in a row, the second smaller; both take the split schedule (the
# first with 256 x 256 pieces, the second with 128 x 128), then a product
# that keeps whole tiles and needs no scratch.
SEQUENCE = [(2047, 2560, 4093, False, False), (768, 640, 6000, True, True), (1024, 1024, 1024, False, True)]


def test_scratch_limit_and_plans():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    limit = sg.sgemm_ex_noalloc_scratch_bytes()
    assert limit == 128 << 20
    need = [sg.sgemm_ex_workspace_size(int(tA), int(tB), M, N, K, cus) for (M, N, K, tA, tB) in SEQUENCE]
    assert 0 < need[1] < need[0] <= limit and need[2] == 0, need


@pytest.mark.parametrize("values", ["pm1", "int"])
def test_noalloc_equals_workspace_entry(values):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for i, (M, N, K, tA, tB) in enumerate(SEQUENCE):
        print(f"[noalloc] {values} call {i}: {M}x{N}x{K} transA={tA} transB={tB}", flush=True)
        if values == "int":
            opA, opB = synth.small_int(90 + i, (M, K)), synth.small_int(95 + i, (K, N))
            C0 = synth.small_int(99 + i, (M, N))
            alpha, beta = 1.0, -2.0
        else:
            opA, opB = synth.operands(M, N, K, "pm1", seed_a=70 + i, seed_b=80 + i)
            C0 = synth.uniform_pm1(60 + i, (M, N))
            alpha, beta = 0.75, 0.5
        A = np.ascontiguousarray(opA.T) if tA else opA
        B = np.ascontiguousarray(opB.T) if tB else opB
        need = sg.sgemm_ex_workspace_size(int(tA), int(tB), M, N, K, cus)
        ws = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device="cuda")  # junk in the workspace
        got = _run("noalloc", M, N, K, A, B, C0, alpha, beta, tA=tA, tB=tB)
        want = _run("ws", M, N, K, A, B, C0, alpha, beta, ws=ws, tA=tA, tB=tB)
        assert np.array_equal(got, want), f"call {i} differs from sgemm_ex_ws"
        if values == "int":
            exact = alpha * (opA.astype(np.float64) @ opB.astype(np.float64)) + beta * C0.astype(np.float64)
            assert np.array_equal(got.astype(np.float64), exact), f"call {i} not exact"
        else:
            rng = np.random.default_rng(i)
            rows = np.concatenate([rng.integers(0, M, 3000), [0, M - 1, M - 1]])
            cols = np.concatenate([rng.integers(0, N, 3000), [N - 1, 0, N - 1]])
            ref, S = oracle.gemm_ex_entries(tA, tB, alpha, A, B, beta, C0, rows, cols)
            assert_within(got[rows, cols], ref, S, f"noalloc call {i}")


def test_checks_and_errors():
    # Host checks come first and match sgemm_ex's; the scratch limit is a
    # clear error where a product would need more than the buffer holds
    # (checked on the host for a device with many more compute units).
    rc = sg.sgemm_ex_noalloc(0, 0, -1, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, None, sg.SGEMM_MFMA)
    assert rc == sg.SGEMM_ERR_DIM
    rc = sg.sgemm_ex_noalloc(0, 0, 0, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, None, sg.SGEMM_MFMA)
    assert rc == sg.SGEMM_OK
    big = sg.sgemm_ex_noalloc_check_args(0, 0, 3001, 2047, 16384, 1.0, 1 << 20, 16384, 1 << 40, 2047, 0.0, 1 << 41,
                                         2047, sg.SGEMM_MFMA, 1024)
    assert big == sg.SGEMM_ERR_SCRATCH
    assert "scratch" in sg.sgemm_status_string(big)
