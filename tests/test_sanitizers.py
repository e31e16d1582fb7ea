"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU tests).

The C ABI's host-only entry points (csrc/args.cpp, csrc/select.cpp) and the C
oracle are rebuilt with g++/gcc and -fsanitize=address,undefined (no GPU code
is involved), then driven over edge-case arguments: sizes from INT_MIN to
INT_MAX, extents at the top of the address space, every transpose pair and
padded leading dimensions on exactly sized buffers. A bad access, a signed
overflow or any other undefined behaviour aborts the driver.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_fp32_matrix_sgemm_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build_and_run(cmd, exe, tmp_path, env_extra=None):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "sanitize" in r.stderr and "unrecognized" in r.stderr:
        pytest.skip("the compiler has no sanitizers")
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               **(env_extra or {}))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, \
        (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_host_entry_points_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", *SAN, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(HERE, "host_checks.cpp"), os.path.join(CSRC, "args.cpp"), os.path.join(CSRC, "select.cpp"),
           "-o", exe]
    assert "host checks ok" in _build_and_run(cmd, exe, tmp_path)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(HERE, "oracle_driver.c"), "-o", exe]
    assert "oracle ok" in _build_and_run(cmd, exe, tmp_path, {"OMP_NUM_THREADS": "2"})
