"""SGEMM_BEST is the fastest rung on every workload (GPU tests).

sgemm_best_variant (include/sgemm.h) names the variant SGEMM_BEST runs for a
shape: the matrix-core kernel, since it measured fastest on every product of
the configuration table. This checks that choice on the GPU: each rung is
timed back to back on the five workloads (the order rotated over rounds, after
a warm-up that brings the chip to its sustained clock), and the variant
sgemm_best_variant names must be within a small margin of the fastest. At 128^3
every rung is bound by its launch (a few microseconds), so the margin there is
wider.
"""

import numpy as np
import pytest
import torch

import dense_fp32_matrix_sgemm_amd as sg
import synth

pytestmark = pytest.mark.gpu

# Margin over the fastest rung's time per workload.
MARGIN = {"sq128": 0.25, "sq1024": 0.05, "sq2048": 0.05, "sq4096": 0.05, "ragged": 0.05}
RUNGS = ["naive", "tiled", "regblock", "mfma"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()


def _time(call, reps):
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        call()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


@pytest.mark.parametrize("workload", list(synth.WORKLOADS))
def test_best_variant_is_the_fastest_rung(workload):
    w = synth.WORKLOADS[workload]
    M, N, K, dist, margin = w["M"], w["N"], w["K"], w["dist"], MARGIN[workload]
    best = sg.sgemm_variant_name(sg.sgemm_best_variant(M, N, K))
    assert best in RUNGS
    print(f"[best] {M}x{N}x{K}: best variant {best}", flush=True)
    A, B = synth.operands(M, N, K, dist)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dC = torch.empty((M, N), device="cuda")
    s = torch.cuda.current_stream()

    def caller(name):
        code = sg.VARIANTS[name]

        def call():
            rc = sg.sgemm(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, s.cuda_stream, code)
            assert rc == sg.SGEMM_OK
        return call

    calls = {name: caller(name) for name in RUNGS}
    # Each rung's launches for about 20 ms per round (at least 3), after a
    # warm-up of the matrix-core kernel for about 50 ms.
    one = {name: _time(calls[name], 1) for name in RUNGS}
    warm = max(3, int(50.0 / max(one["mfma"], 1e-3)))
    _time(calls["mfma"], warm)
    times = {name: [] for name in RUNGS}
    for r in range(3):
        order = RUNGS[r:] + RUNGS[:r]
        for name in order:
            reps = max(3, min(2000, int(20.0 / max(one[name], 1e-3))))
            times[name].append(_time(calls[name], reps))
    med = {name: float(np.median(v)) for name, v in times.items()}
    fastest = min(med, key=med.get)
    print(f"[best] {M}x{N}x{K}: " + ", ".join(f"{n} {1e3 * med[n]:.1f} us" for n in RUNGS), flush=True)
    assert med[best] <= (1.0 + margin) * med[fastest], (best, med)
