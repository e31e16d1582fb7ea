#!/usr/bin/env python3
"""FP32 SGEMM throughput on one MI355X: TFLOP/s at M = N = K = 4096 and the
fraction of the chip's FP32 peak.

One step is one call of the library's C ABI computing C = A * B for the
4096^3 workload (row-major float32, A and B i.i.d. on [0, 1) from seeded
SplitMix64), with A, B and C resident in HBM before timing starts. W untimed
warm-up steps, then K steps timed with HIP events on the stream the kernel is
launched on. Prints one JSON line on stdout; progress goes to stderr.

Also reported:
  roofline      the kernel's achieved TFLOP/s (2 M N K per launch over the
                mean launch duration) against the FP32 matrix peak, and the
                HBM traffic measured with rocprofv3 counters when it is on
                file for the current kernel source;
  cpu_baseline  the CPU oracle (double-accumulating triple loop, OpenMP) timed
                on a bounded sample of the same product on the host cores;
  ladder        every kernel variant timed on the same workload (run before
                the headline, which it also brings to the chip's sustained
                clock: from idle the clock needs about 30 ms of load);
  general_form  the best variant on the same sizes as C = alpha * op(A) *
                op(B) + beta * C, for every transpose pair with beta 0 and 1;
  lowp          the reduced-precision workload (bf16 and f16 operands, FP32
                accumulation) on the same sizes, against the 16-bit matrix
                peak, with sampled elements checked against the oracle;
  check         sampled elements compared with the oracle, and the
                whole-matrix sum of C in double;
  configs       the same entry point and variant on the other workloads of
                the configuration table (128^3, 1024^3, 2048^3 and the ragged
                3001 x 2047 x 4093 on U[-1, 1)): mean per-launch time,
                TFLOP/s, fraction of peak and a sampled oracle check each.

With --cold it instead times the product with the caches flushed by a 512 MiB
write before every launch, next to the same launches back to back.

With --all-configs it instead times every kernel variant on every workload of
the method's configuration table (128^3, 1024^3, 2048^3, 4096^3 and the ragged
3001 x 2047 x 4093 on U[-1, 1)): median and minimum launch time, each result
checked on sampled elements (and the matrix-core variant through sgemm_ex_ws
where the library would split the product), the CPU oracle timed on each whole
product (and on one thread at 128^3 and 1024^3), and the shader clock read
before and after.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks. 157.3 TFLOP/s is the FP32 figure for both the
# matrix cores and the vector ALUs (256 CUs x 256 FLOP/clk x 2.4 GHz); the
# scalar-FMA rungs are rated against it too (they run measurably above half
# of it, so half is not their ceiling).
PEAK_FP32_TFLOPS = 157.3
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 / fp16 matrix peak (the reduced-precision workload)
PEAK_HBM_GBS = 8000.0

METRIC = "FP32 SGEMM TFLOP/s at 4096^3 on 1 MI355X; % of FP32 peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mfma_sq4096_traffic.json")
KERNEL_SOURCES = ["mfma.hpp", "wsplit.hpp", "mfma_nn.hip", "tile_io.hpp", "gemm.hpp", "tiles.hpp", "select.cpp"]


def flops(M: int, N: int, K: int) -> int:
    """Algorithmic FLOP of one product: K multiplies and K adds per element
    of C ("Matrix Multiplication -- Naive to Tiled", section 03)."""
    return 2 * M * N * K


def compulsory_bytes(M: int, N: int, K: int) -> int:
    """Bytes that must cross HBM at least once: read A and B, write C."""
    return 4 * (M * K + K * N + M * N)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dense_fp32_matrix_sgemm_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_per_launch():
    """HBM bytes per launch from the committed counter runs, or None when they
    are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_launches(call, steps: int, warmup: int, per_launch: bool = True):
    """Warm up, then time `steps` back-to-back launches with HIP events on the
    launch stream. Returns (total ms, list of per-launch ms, or None).

    With per_launch, an event is recorded between consecutive launches, which
    gives each launch's interval but adds the events' own cost to it (a few
    microseconds a launch, a tenth of a 1024^3 product). Without, the events
    bracket the whole run only, so the launches follow each other as a
    caller's would, and the mean launch time is total / steps."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    if not per_launch:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), None
    events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    events[0].record(stream)
    for i in range(steps):
        call()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [events[i].elapsed_time(events[i + 1]) for i in range(steps)]
    return events[0].elapsed_time(events[steps]), per


FLUSH_BYTES = 512 << 20  # twice the 256 MB Infinity Cache; each XCD's 4 MB L2 goes with it


def cold_cache(call, M: int, N: int, K: int, args, dev):
    """The product with cold caches: before every timed launch a 512 MiB
    buffer is written on the same stream, which evicts A, B and C from the L2
    and the Infinity Cache, and HIP events bracket the product alone. The same
    launches back to back (hot) are timed beside it."""
    import torch
    stream = torch.cuda.current_stream()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        call()
    cold = []
    for i in range(args.steps):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    _, hot = time_launches(call, args.steps, 1)
    f = flops(M, N, K)
    res = {"config": {"M": M, "N": N, "K": K}, "flush_bytes": FLUSH_BYTES, "steps": args.steps}
    for name, v in (("cold", cold), ("hot", hot)):
        mean = sum(v) / len(v)
        res[name] = {"kernel_ms_mean": round(mean, 5), "kernel_ms_min": round(min(v), 5),
                     "TFLOP/s": round(f / (mean / 1e3) / 1e12, 3),
                     "frac": round(f / (mean / 1e3) / 1e12 / PEAK_FP32_TFLOPS, 4)}
    log(f"cold {res['cold']['kernel_ms_mean']:.4f} ms, hot {res['hot']['kernel_ms_mean']:.4f} ms")
    return res


def cpu_baseline(A, B, target_s: float):
    """The oracle on the first R rows of the product, R sized for about
    target_s seconds of host time (at least 64 rows)."""
    import numpy as np
    import oracle
    M, K = A.shape
    N = B.shape[1]
    probe = min(M, 64)
    t0 = time.perf_counter()
    oracle.gemm(np.ascontiguousarray(A[:probe]), B)
    dt = time.perf_counter() - t0
    rows = int(min(M, max(probe, probe * target_s / max(dt, 1e-6))))
    rows = max(probe, rows - rows % 8) if rows < M else M
    t0 = time.perf_counter()
    oracle.gemm(np.ascontiguousarray(A[:rows]), B)
    dt = time.perf_counter() - t0
    out = {
        "value": round(flops(rows, N, K) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of the {M}x{N}x{K} product "
                  f"({rows / M:.3f} of its work), {dt:.1f} s",
        "cpu_model": cpu_model(),
    }
    # The same oracle on one host thread at the two smaller square sizes.
    one = {}
    for n in (128, 1024):
        try:
            s1 = oracle_seconds_one_thread(n, n, n, "u01")
        except Exception as e:  # a baseline only: report, do not fail the bench
            one[f"{n}^3"] = {"error": str(e)[:200]}
            continue
        one[f"{n}^3"] = {"seconds": round(s1, 4), "TFLOP/s": round(flops(n, n, n) / s1 / 1e12, 6)}
    out["one_thread"] = one
    return out


def cpu_model() -> str | None:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# The method's configuration table: (M, N, K, value distribution).
CONFIGS = [(128, 128, 128, "u01"), (1024, 1024, 1024, "u01"), (2048, 2048, 2048, "u01"),
           (4096, 4096, 4096, "u01"), (3001, 2047, 4093, "pm1")]


# Variants timed by --all-configs: the four rungs (the tiled one with the tile
# size it picks for the shape) and the tiled rung at each fixed T.
ALL_CONFIG_VARIANTS = ("naive", "tiled", "tiled8", "tiled16", "tiled32", "regblock", "mfma")


def read_sclk():
    """Current shader clock level of each GPU as the driver reports it (the
    starred line of pp_dpm_sclk), or None where the file is not readable."""
    import glob
    out = {}
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                cur = [line.strip() for line in f if line.strip().endswith("*")]
        except OSError:
            continue
        out[path.split("/")[4]] = cur[0] if cur else None
    return out or None


def oracle_seconds_one_thread(M: int, N: int, K: int, dist: str) -> float:
    """The oracle on one host thread, in a child process (its OpenMP thread
    count is fixed at start-up)."""
    import subprocess
    code = ("import sys, time, synth, oracle\n"
            f"A, B = synth.operands({M}, {N}, {K}, '{dist}')\n"
            "t0 = time.perf_counter(); oracle.gemm(A, B); print(time.perf_counter() - t0)\n")
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600, check=True)
    return float(r.stdout.strip().splitlines()[-1])


def all_configs(lib, sg, dev, only=None) -> dict:
    """Every variant on every configuration (or the variants named in
    `only`): timing, sampled check, oracle."""
    import numpy as np
    import torch

    import oracle
    import synth
    from oracle.check import excess
    stream = torch.cuda.current_stream()
    result = {"sclk_before": read_sclk(), "oracle_threads": oracle.num_threads(), "configs": []}
    for (M, N, K, dist) in CONFIGS:
        log(f"all-configs: {M}x{N}x{K} ({dist})")
        A, B = synth.operands(M, N, K, dist)
        dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        dC = torch.zeros((M, N), dtype=torch.float32, device=dev)
        f = flops(M, N, K)
        rng = np.random.default_rng(M + N + K)
        rows = np.concatenate([[0, M - 1], rng.integers(0, M, 1022)])
        cols = np.concatenate([[N - 1, 0], rng.integers(0, N, 1022)])
        ref, sabs = oracle.gemm_entries(A, B, rows, cols)
        entry = {"M": M, "N": N, "K": K, "values": dist, "variants": {}}
        for name in ALL_CONFIG_VARIANTS:
            if only is not None and name not in only:
                continue
            code = sg.VARIANTS[name]

            def call(code=code):
                rc = lib.sgemm(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
                               stream.cuda_stream, code)
                if rc != 0:
                    raise sg.SgemmError(rc)
            dC.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            worst = float(excess(dC.cpu().numpy()[rows, cols], ref, sabs).max())
            t0 = time.perf_counter()
            call()
            torch.cuda.synchronize()
            one = time.perf_counter() - t0
            reps = int(max(50, min(2000, 0.1 / max(one, 1e-6))))
            tot, _ = time_launches(call, reps, 3, per_launch=False)
            _, per = time_launches(call, reps, 1)
            med, mn = float(np.median(per)), min(per)
            entry["variants"][name] = {
                "reps": reps, "ms_mean_back_to_back": round(tot / reps, 5),
                "ms_median": round(med, 5), "ms_min": round(mn, 5),
                "TFLOP/s_median": round(f / (med / 1e3) / 1e12, 3), "TFLOP/s_max": round(f / (mn / 1e3) / 1e12, 3),
                "frac_of_fp32_peak_median": round(f / (med / 1e3) / 1e12 / PEAK_FP32_TFLOPS, 4),
                "check_worst_error_over_bound": round(worst, 4)}
            log(f"  {name}: median {med:.4f} ms, min {mn:.4f} ms, "
                f"{entry['variants'][name]['TFLOP/s_median']} TFLOP/s, check {worst:.3f}")
        # The matrix-core variant through sgemm_ex_ws, where the library puts
        # the product on its split schedule.
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        need = sg.sgemm_ex_workspace_size(sg.SGEMM_OP_N, sg.SGEMM_OP_N, M, N, K, cus)
        if need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)

            def call_ws():
                rc = lib.sgemm_ex_ws(0, 0, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, dC.data_ptr(), N,
                                     ws.data_ptr(), need, stream.cuda_stream, sg.SGEMM_MFMA)
                if rc != 0:
                    raise sg.SgemmError(rc)
            dC.fill_(float("nan"))
            call_ws()
            torch.cuda.synchronize()
            worst = float(excess(dC.cpu().numpy()[rows, cols], ref, sabs).max())
            _, per = time_launches(call_ws, 100, 3)
            med, mn = float(np.median(per)), min(per)
            entry["variants"]["mfma_split"] = {
                "reps": 100, "workspace_bytes": need, "ms_median": round(med, 5), "ms_min": round(mn, 5),
                "TFLOP/s_median": round(f / (med / 1e3) / 1e12, 3), "TFLOP/s_max": round(f / (mn / 1e3) / 1e12, 3),
                "frac_of_fp32_peak_median": round(f / (med / 1e3) / 1e12 / PEAK_FP32_TFLOPS, 4),
                "check_worst_error_over_bound": round(worst, 4)}
            log(f"  mfma_split: median {med:.4f} ms, {entry['variants']['mfma_split']['TFLOP/s_median']} TFLOP/s, "
                f"check {worst:.3f}")
            del ws
        t0 = time.perf_counter()
        oracle.gemm(A, B)
        dt = time.perf_counter() - t0
        entry["oracle"] = {"seconds": round(dt, 4), "TFLOP/s": round(f / dt / 1e12, 6)}
        if M in (128, 1024) and M == N == K:
            dt1 = oracle_seconds_one_thread(M, N, K, dist)
            entry["oracle_one_thread"] = {"seconds": round(dt1, 4), "TFLOP/s": round(f / dt1 / 1e12, 6)}
        result["configs"].append(entry)
        del dA, dB, dC
    result["sclk_after"] = read_sclk()
    return result


def config_sweep(lib, sg, dev, variant: int) -> dict:
    """The product on the other workloads of the configuration table, through
    the same entry point and variant as the headline: per-launch HIP-event
    times of back-to-back launches (warm-up first), and 1024 sampled elements
    (the four corners included) checked against the oracle."""
    import numpy as np
    import torch

    import oracle
    import synth
    from oracle.check import excess, within
    stream = torch.cuda.current_stream()
    out = {}
    for (M, N, K, dist) in CONFIGS:
        if (M, N, K) == (4096, 4096, 4096):
            continue  # the headline
        A, B = synth.operands(M, N, K, dist)
        dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        dC = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
        resolved = sg.sgemm_best_variant(M, N, K) if variant == sg.SGEMM_BEST else variant

        def call():
            rc = lib.sgemm(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, stream.cuda_stream,
                           variant)
            if rc != 0:
                raise sg.SgemmError(rc)
        call()
        torch.cuda.synchronize()
        rng = np.random.default_rng(M + 2 * N + 3 * K)
        rows = np.concatenate([[0, 0, M - 1, M - 1], rng.integers(0, M, 1020)])
        cols = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 1020)])
        ref, sabs = oracle.gemm_entries(A, B, rows, cols)
        got = dC.cpu().numpy()[rows, cols]
        t0 = time.perf_counter()
        call()
        torch.cuda.synchronize()
        one = time.perf_counter() - t0
        reps = int(max(50, min(2000, 0.2 / max(one, 1e-6))))
        # Warm-up long enough (about 50 ms of launches) for the clock to settle.
        total, _ = time_launches(call, reps, int(max(20, min(4000, 0.05 / max(one, 1e-6)))), per_launch=False)
        mean = total / reps
        _, per = time_launches(call, min(reps, 200), 5)
        med = float(np.median(per))
        f = flops(M, N, K)
        tf = f / (mean / 1e3) / 1e12
        key = f"{M}x{N}x{K}"
        out[key] = {"values": dist, "variant": sg.sgemm_variant_name(resolved), "reps": reps,
                    "kernel_ms_mean": round(mean, 5), "kernel_ms_median_with_events_between": round(med, 5),
                    "TFLOP/s": round(tf, 3), "frac": round(tf / PEAK_FP32_TFLOPS, 4),
                    "check_sampled_elements": int(rows.size),
                    "check_worst_error_over_bound": round(float(excess(got, ref, sabs).max()), 4),
                    "check_pass": bool(within(got, ref, sabs).all())}
        if resolved == sg.SGEMM_MFMA:
            out[key]["mfma_tile"] = "x".join(str(v) for v in sg.sgemm_mfma_shape(M, N, K)[:3])
        log(f"config {key}: {mean:.4f} ms mean, {tf:.2f} TFLOP/s, check {out[key]['check_worst_error_over_bound']}")
        del dA, dB, dC
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--variant", default="best",
                    choices=["best", "naive", "tiled", "tiled8", "tiled16", "tiled32", "regblock", "mfma"])
    ap.add_argument("--size", type=int, default=4096, help="M = N = K")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ladder", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-general-form", action="store_true")
    ap.add_argument("--no-lowp", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads of the configuration table")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="host time budget of the CPU-baseline sample")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the headline, time every variant on every configuration "
                         "and the CPU oracle on each")
    ap.add_argument("--only", default=None,
                    help="with --all-configs: comma-separated variants to run (default: all of " +
                         ", ".join(ALL_CONFIG_VARIANTS) + ")")
    ap.add_argument("--cold", action="store_true",
                    help="instead of the headline line, time the product with the caches flushed "
                         "(a 512 MiB write) before every launch, next to the same launches back to back")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the product, time a plain 256 MiB device copy "
                         "(reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU: this build has no multi-GPU path "
               f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})")
        print(msg, file=sys.stderr)
        if int(os.environ.get("RANK", "0")) == 0:
            print(json.dumps({"metric": METRIC, "error": msg, "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import dense_fp32_matrix_sgemm_amd as sg
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    lib = sg.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 64 << 20  # floats: 256 MiB
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        total, per = time_launches(lambda: dst.copy_(src), args.steps, args.warmup)
        ms = total / args.steps
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                          "ms_per_copy": round(ms, 5),
                          "GB_per_s": round(8 * n / (ms / 1e3) / 1e9, 1)}))
        return 0

    if args.all_configs:
        only = None
        if args.only:
            only = set(args.only.split(","))
            unknown = only - set(ALL_CONFIG_VARIANTS)
            if unknown:
                print(f"--only: unknown variants {sorted(unknown)}", file=sys.stderr)
                return 2
        print(json.dumps({"metric": METRIC, "all_configs": all_configs(lib, sg, dev, only)}), flush=True)
        return 0

    M = N = K = args.size
    log(f"generating {M}x{K} and {K}x{N} inputs")
    A, B = synth.operands(M, N, K, "u01")
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.zeros((M, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    variant = sg.VARIANTS[args.variant]
    resolved = sg.sgemm_best_variant(M, N, K) if variant == sg.SGEMM_BEST else variant
    stream = torch.cuda.current_stream()
    pa, pb, pc = dA.data_ptr(), dB.data_ptr(), dC.data_ptr()

    def make_call(v):
        def call():
            rc = lib.sgemm(M, N, K, pa, K, pb, N, pc, N, stream.cuda_stream, v)
            if rc != 0:
                raise sg.SgemmError(rc)
        return call

    if args.cold:
        print(json.dumps({"metric": METRIC, "cold_cache": cold_cache(make_call(variant), M, N, K, args, dev)}),
              flush=True)
        return 0

    # The ladder (every rung on the same workload) runs before the headline:
    # besides its own figures it keeps the chip busy for about a second, so
    # that the headline's warm-up and timed steps start at the clock the chip
    # holds under sustained load. From idle the clock takes about 30 launches
    # of this product (30 ms) to settle, which a few warm-up steps do not cover.
    f = flops(M, N, K)
    ladder = None
    if not args.no_ladder:
        ladder = {}
        for name in ("naive", "tiled", "regblock", "mfma"):
            code = sg.VARIANTS[name]
            call = make_call(code)
            call()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            call()
            torch.cuda.synchronize()
            one = time.perf_counter() - t0
            reps = max(3, min(50, int(0.5 / max(one, 1e-6))))
            tot, _ = time_launches(call, reps, 1, per_launch=False)
            vms = tot / reps
            tf = f / (vms / 1e3) / 1e12
            ladder[name] = {"ms": round(vms, 4), "TFLOP/s": round(tf, 3),
                            "pct_of_fp32_peak": round(100 * tf / PEAK_FP32_TFLOPS, 2),
                            "bound": "mfma" if code == sg.SGEMM_MFMA else "alu", "reps": reps}
            log(f"ladder {name}: {vms:.3f} ms, {tf:.2f} TFLOP/s")

    log(f"timing {args.steps} steps of variant {sg.sgemm_variant_name(resolved)} "
        f"after {args.warmup} warm-up steps")
    total_ms, _ = time_launches(make_call(variant), args.steps, args.warmup, per_launch=False)
    ms = total_ms / args.steps
    kernel_ms = ms  # back-to-back launches: the mean launch time
    f = flops(M, N, K)
    value = f / (ms / 1e3) / 1e12
    achieved = f / (kernel_ms / 1e3) / 1e12
    bound_peak = PEAK_FP32_TFLOPS
    log(f"{ms:.4f} ms/step, {value:.2f} TFLOP/s ({100 * value / PEAK_FP32_TFLOPS:.1f}% of "
        f"{PEAK_FP32_TFLOPS} peak)")

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "pct_of_fp32_peak": round(100 * value / PEAK_FP32_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"sgemm C=A*B, M=N=K={M}, row-major float32, A,B i.i.d. U[0,1) "
                        "(SplitMix64 seeds 42/43), C overwritten",
            "M": M, "N": N, "K": K,
            "variant": sg.sgemm_variant_name(resolved),
        },
        "roofline": {
            "bound": "mfma" if resolved == sg.SGEMM_MFMA else "alu",
            "achieved": round(achieved, 3),
            "peak": bound_peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / bound_peak, 4),
            "traffic": traffic_per_launch() if (M == 4096 and resolved == sg.SGEMM_MFMA) else None,
            "kernel_ms_mean": round(kernel_ms, 5),
            "compulsory_bytes": compulsory_bytes(M, N, K),
        },
    }

    if not args.no_check:
        import oracle
        from oracle.check import excess, within
        torch.cuda.synchronize()
        C = dC.cpu().numpy()
        rng = np.random.default_rng(1)
        rows = np.concatenate([[0, 0, M - 1, M - 1], rng.integers(0, M, 2044)])
        cols = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 2044)])
        ref, sabs = oracle.gemm_entries(A, B, rows, cols)
        worst = float(excess(C[rows, cols], ref, sabs).max())
        out["check"] = {
            "sampled_elements": int(rows.size),
            "worst_error_over_bound": round(worst, 4),
            "pass": bool(within(C[rows, cols], ref, sabs).all()),
            "checksum_sum_C_double": float(C.astype(np.float64).sum()),
        }
        log(f"check: {rows.size} sampled elements, worst error {worst:.3f} of bound")

    if ladder is not None:
        out["ladder"] = ladder

    if not args.no_configs:
        out["configs"] = config_sweep(lib, sg, dev, variant)

    if not args.no_general_form:
        # Same sizes, stored transposed where the pair says so; alpha = 1.
        # With beta = 0 every pair sums each element in the same order as
        # the plain call, so its C must equal the plain C bit for bit.
        torch.cuda.synchronize()
        plain = dC.clone()
        dAt, dBt = dA.t().contiguous(), dB.t().contiguous()
        dC2 = torch.empty_like(dC)
        general = {}
        for ta in (0, 1):
            for tb in (0, 1):
                pa2, lda2 = (dAt.data_ptr(), M) if ta else (pa, K)
                pb2, ldb2 = (dBt.data_ptr(), K) if tb else (pb, N)
                for beta in (0.0, 1.0):
                    dC2.copy_(plain)

                    def call(ta=ta, tb=tb, pa2=pa2, lda2=lda2, pb2=pb2, ldb2=ldb2, beta=beta):
                        rc = lib.sgemm_ex(ta, tb, M, N, K, 1.0, pa2, lda2, pb2, ldb2, beta,
                                          dC2.data_ptr(), N, stream.cuda_stream, variant)
                        if rc != 0:
                            raise sg.SgemmError(rc)
                    if beta == 0.0:
                        call()
                        torch.cuda.synchronize()
                        same = bool(torch.equal(dC2, plain))
                    tot, _ = time_launches(call, 50, 10, per_launch=False)
                    kms = tot / 50
                    key = ("t" if ta else "n") + ("t" if tb else "n") + f"_beta{int(beta)}"
                    general[key] = {"kernel_ms_mean": round(kms, 5),
                                    "TFLOP/s": round(f / (kms / 1e3) / 1e12, 3),
                                    "frac": round(f / (kms / 1e3) / 1e12 / PEAK_FP32_TFLOPS, 4)}
                    if beta == 0.0:
                        general[key]["bitwise_equal_to_plain"] = same
                    log(f"general form {key}: {kms:.4f} ms, {general[key]['TFLOP/s']} TFLOP/s")
        out["general_form"] = general
        del dAt, dBt, dC2, plain

    if not args.no_lowp:
        import oracle
        from oracle.check import excess
        lowp = {}
        rng = np.random.default_rng(2)
        rows, cols = rng.integers(0, M, 256), rng.integers(0, N, 256)
        for dt in ("bf16", "f16"):
            Av = synth.lowp_values(synth.SEED_A, (M, K), dt)
            Bv = synth.lowp_values(synth.SEED_B, (K, N), dt)
            Ab, Bb = synth.to_lowp_bits(Av, dt), synth.to_lowp_bits(Bv, dt)
            Bt = np.ascontiguousarray(Bb.T)
            dAl = torch.from_numpy(Ab.view(np.int16)).to(dev)
            for pair, Bst in (("nn", Bb), ("nt", Bt)):
                dBl = torch.from_numpy(Bst.view(np.int16)).to(dev)
                tb = 1 if pair == "nt" else 0

                def call(dBl=dBl, tb=tb):
                    rc = lib.sgemm_lp(sg.LP_TYPES[dt], 0, tb, M, N, K, 1.0, dAl.data_ptr(), K, dBl.data_ptr(),
                                      K if tb else N, 0.0, dC.data_ptr(), N, stream.cuda_stream)
                    if rc != 0:
                        raise sg.SgemmError(rc)
                tot, _ = time_launches(call, 50, 10, per_launch=False)
                kms = tot / 50
                tf = f / (kms / 1e3) / 1e12
                torch.cuda.synchronize()
                Cl = dC.cpu().numpy()
                ref, sabs = oracle.gemm_entries(oracle.lowp_to_float32(Ab, dt), oracle.lowp_to_float32(Bb, dt),
                                                rows, cols)
                worst = float(excess(Cl[rows, cols], ref, sabs).max())
                lowp[f"{dt}_{pair}"] = {"kernel_ms_mean": round(kms, 5), "TFLOP/s": round(tf, 2),
                                        "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                        "check_worst_error_over_bound": round(worst, 4)}
                log(f"lowp {dt} {pair}: {kms:.4f} ms, {tf:.1f} TFLOP/s, check {worst:.3f}")
                del dBl
            del dAl
        out["lowp"] = lowp

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the product")
        out["cpu_baseline"] = cpu_baseline(A, B, args.cpu_seconds)
        log(f"cpu baseline: {out['cpu_baseline']}")

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
