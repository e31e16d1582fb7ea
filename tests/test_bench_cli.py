"""bench.py's command-line contract and its host-side helpers (CPU tests)."""

import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "error" in line


def test_distributed_launch_is_refused_on_every_rank():
    env = dict(os.environ, WORLD_SIZE="2", RANK="1")
    r = _run(env=env)
    assert r.returncode == 2
    assert r.stdout.strip() == ""           # only rank 0 prints the JSON line


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES") is None and os.path.exists("/dev/kfd"),
                    reason="a GPU may be present")
def test_without_a_gpu_it_fails_loudly():
    r = _run("--no-cpu-baseline")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr


def test_work_and_bytes():
    assert bench.flops(4096, 4096, 4096) == 2 * 4096**3
    assert bench.flops(3001, 2047, 4093) == 2 * 3001 * 2047 * 4093
    assert bench.compulsory_bytes(4096, 4096, 4096) == 4 * 3 * 4096**2 == 201326592


def test_configuration_table():
    # 128^3 .. 4096^3 on U[0,1) and the ragged 3001 x 2047 x 4093 on U[-1,1).
    assert bench.CONFIGS == [(128, 128, 128, "u01"), (1024, 1024, 1024, "u01"), (2048, 2048, 2048, "u01"),
                             (4096, 4096, 4096, "u01"), (3001, 2047, 4093, "pm1")]


def test_clock_reader_never_raises():
    s = bench.read_sclk()
    assert s is None or all(isinstance(k, str) for k in s)


def test_traffic_is_only_reported_for_the_profiled_source():
    t = bench.traffic_per_launch()
    with open(bench.TRAFFIC_FILE) as f:
        on_file = json.load(f)
    if on_file["kernel_source_hash"] == bench.kernel_source_hash():
        assert t == on_file["bytes_per_launch"]
    else:
        assert t is None
