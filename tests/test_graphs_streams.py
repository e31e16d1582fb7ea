"""The entry points under HIP graph capture and on concurrent streams (GPU).

Every entry point only enqueues kernels: no allocation, no memset, no host
synchronisation. So a sequence of calls can be captured in a HIP graph and
replayed, which is how a launch-bound caller would use it. Each replay here
runs on new input values copied into the captured buffers, with eager work
and a synchronisation between replays, and every replay is checked against
the oracle. Calls on two streams at once must not interfere.
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


def test_graph_capture_and_replay():
    print("[graphs] capture and replay", flush=True)
    dev = torch.device("cuda:0")
    M, N, K = 300, 260, 333
    dA = torch.empty((M, K), device=dev)
    dB = torch.empty((K, N), device=dev)
    dBt = torch.empty((N, K), device=dev)
    dC1 = torch.empty((M, N), device=dev)
    dC2 = torch.empty((M, N), device=dev)
    dAl = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dBl = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
    dC3 = torch.empty((M, N), device=dev)

    def work():
        sg.matmul(dA, dB, out=dC1)                         # sgemm
        sg.gemm(dA, dBt.t(), dC2, alpha=-0.5, beta=1.5)    # sgemm_ex, B transposed, C read
        sg.gemm(dAl, dBl, dC3)                             # sgemm_lp

    def load(seed):
        A, B = synth.operands(M, N, K, "pm1", seed_a=seed, seed_b=seed + 1)
        C2 = synth.uniform_pm1(seed + 2, (M, N))
        Al = synth.lowp_values(seed + 3, (M, K), "bf16", "pm1")
        Bl = synth.lowp_values(seed + 4, (K, N), "bf16", "pm1")
        dA.copy_(torch.from_numpy(A))
        dB.copy_(torch.from_numpy(B))
        dBt.copy_(torch.from_numpy(np.ascontiguousarray(B.T)))
        dC2.copy_(torch.from_numpy(C2))
        dAl.copy_(torch.from_numpy(Al).to(torch.bfloat16))
        dBl.copy_(torch.from_numpy(Bl).to(torch.bfloat16))
        return A, B, C2, Al, Bl

    def check(data, what):
        A, B, C2, Al, Bl = data
        Cref, S = oracle.gemm(A, B, with_abs=True)
        assert_within(dC1.cpu().numpy(), Cref, S, f"{what} sgemm")
        Cref, S = oracle.gemm_ex(False, True, -0.5, A, np.ascontiguousarray(B.T), 1.5, C2)
        assert_within(dC2.cpu().numpy(), Cref, S, f"{what} sgemm_ex")
        Cref, S = oracle.gemm(Al, Bl, with_abs=True)
        assert_within(dC3.cpu().numpy(), Cref, S, f"{what} sgemm_lp")

    side = torch.cuda.Stream()
    data = load(10)
    with torch.cuda.stream(side):       # warm-up off the capture
        work()
    torch.cuda.synchronize()
    check(data, "eager")

    graph = torch.cuda.CUDAGraph()
    data = load(20)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        data = load(30 + 10 * rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check(data, f"replay {rep}")
        # Eager work between replays.
        torch.matmul(dA, dB).sum().item()
    del graph


def test_two_streams_at_once():
    print("[graphs] two streams", flush=True)
    dev = torch.device("cuda:0")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cases = []
    for i, (M, N, K) in enumerate([(1500, 1300, 1100), (700, 900, 2100)]):
        A, B = synth.operands(M, N, K, "pm1", seed_a=50 + i, seed_b=60 + i)
        cases.append((A, B, torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                      torch.empty((M, N), device=dev)))
    torch.cuda.synchronize()
    for _ in range(5):
        with torch.cuda.stream(s1):
            sg.matmul(cases[0][2], cases[0][3], out=cases[0][4])
        with torch.cuda.stream(s2):
            sg.matmul(cases[1][2], cases[1][3], out=cases[1][4])
    torch.cuda.synchronize()
    for A, B, _, _, dC in cases:
        Cref, S = oracle.gemm(A, B, with_abs=True)
        assert_within(dC.cpu().numpy(), Cref, S, "two streams")


def test_split_schedule_under_graph_capture():
    # sgemm_ex_ws on the split schedule (two kernels and the workspace, no
    # allocation and no memset) captured once and replayed on new inputs.
    print("[graphs] split schedule capture and replay", flush=True)
    dev = torch.device("cuda:0")
    M, N, K = 1000, 1000, 8000
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    need = sg.sgemm_ex_workspace_size(sg.SGEMM_OP_N, sg.SGEMM_OP_N, M, N, K, cus)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    dA = torch.empty((M, K), device=dev)
    dB = torch.empty((K, N), device=dev)
    dC = torch.empty((M, N), device=dev)
    rng = np.random.default_rng(7)
    rows, cols = rng.integers(0, M, 2000), rng.integers(0, N, 2000)

    def load(seed):
        A, B = synth.operands(M, N, K, "pm1", seed_a=seed, seed_b=seed + 1)
        C0 = synth.uniform_pm1(seed + 2, (M, N))
        dA.copy_(torch.from_numpy(A))
        dB.copy_(torch.from_numpy(B))
        dC.copy_(torch.from_numpy(C0))
        return A, B, C0

    def check(data, what):
        A, B, C0 = data
        want, S = oracle.gemm_ex_entries(False, False, 1.5, A, B, -0.5, C0, rows, cols)
        assert_within(dC.cpu().numpy()[rows, cols], want, S, what)

    side = torch.cuda.Stream()
    data = load(60)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        sg.gemm(dA, dB, dC, alpha=1.5, beta=-0.5, workspace=ws)
    torch.cuda.synchronize()
    check(data, "eager")
    graph = torch.cuda.CUDAGraph()
    load(70)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        sg.gemm(dA, dB, dC, alpha=1.5, beta=-0.5, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        data = load(80 + 10 * rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check(data, f"replay {rep}")
        torch.matmul(dA, dB).sum().item()   # eager work between replays
    del graph


def test_host_threads_each_with_a_stream():
    # The library keeps no per-call state and only a per-device cache of the
    # architecture (an atomic per device), so host threads may call it at
    # once, each on its own stream.
    import threading
    print("[graphs] four host threads", flush=True)
    dev = torch.device("cuda:0")
    shapes = [(700, 900, 500), (1024, 1024, 1024), (333, 2049, 777), (1500, 600, 1100)]
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = synth.operands(M, N, K, "pm1", seed_a=70 + i, seed_b=80 + i)
        data.append((A, B, torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                     [torch.empty((M, N), device=dev) for _ in range(3)]))
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            _, _, dA, dB, outs = data[i]
            with torch.cuda.stream(s):
                for rep in range(12):
                    sg.matmul(dA, dB, out=outs[rep % 3])
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for A, B, _, _, outs in data:
        Cref, S = oracle.gemm(A, B, with_abs=True)
        for dC in outs:
            assert_within(dC.cpu().numpy(), Cref, S, "host threads")
