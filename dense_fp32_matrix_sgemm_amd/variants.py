"""Build variants of the library with other tile settings and time them.

The tile shapes, register sets, wave counts and band height of the matrix
kernels are preprocessor macros with defaults (``csrc/tiles.hpp``,
``csrc/lowp.hpp``; ``SGEMM_MFMA_FORCE_TILE`` in ``csrc/select.cpp`` pins the
tile choice), so a sweep over them is a set of builds of the same sources:

    python -m dense_fp32_matrix_sgemm_amd.variants build OUT/w32 -DSGEMM_MFMA_WSPLIT64="2, 16, 2, 2"
    python -m dense_fp32_matrix_sgemm_amd.variants time cur=dense_fp32_matrix_sgemm_amd/lib/libsgemm.so,w32=OUT/w32/libsgemm.so 1024x1024x1024,2048x2048x2048:2048:2048

``build`` compiles every source with the extra hipcc arguments into
``OUT/<name>/libsgemm.so`` (objects in ``OUT/<name>/obj``). ``time`` runs
``sgemm`` (row-major, C = A*B) of each library on the same device operands,
in five interleaved rounds of back-to-back launches after the chip has been
brought to its sustained clock, and prints each library's median time and
TFLOP/s per shape. Shapes are ``MxNxK`` with optional ``:lda:ldb``. Before
timing, every library's result is compared with a float64 product of the same
operands on the device: the worst |C - AB| over (K 2^-24 |A||B| + 1e-30) is
printed beside the time, and a value of 1 or more stops the run, so a variant
that computes the wrong product is never reported as faster.
"""

from __future__ import annotations

import ctypes
import os
import sys

from . import _build


def build_variant(out_dir: str, hipcc_args: list[str]) -> str:
    """Compile the library with extra hipcc arguments into out_dir; returns the path."""
    out_dir = os.path.abspath(out_dir)
    saved = (_build.HIPCC_FLAGS, _build.OBJDIR, _build.LIBDIR, _build.LIB_PATH)
    try:
        _build.HIPCC_FLAGS = list(saved[0]) + list(hipcc_args)
        _build.OBJDIR = os.path.join(out_dir, "obj")
        _build.LIBDIR = out_dir
        _build.LIB_PATH = os.path.join(out_dir, "libsgemm.so")
        return _build.build()
    finally:
        _build.HIPCC_FLAGS, _build.OBJDIR, _build.LIBDIR, _build.LIB_PATH = saved


def _parse_shape(spec: str):
    dims, *lds = spec.split(":")
    M, N, K = (int(x) for x in dims.split("x"))
    if min(M, N, K) <= 0:
        raise ValueError(f"shape {spec}: sizes must be positive")
    lda = int(lds[0]) if lds else K
    ldb = int(lds[1]) if len(lds) > 1 else N
    if lda < K or ldb < N:
        raise ValueError(f"shape {spec}: leading dimensions below the row lengths")
    return M, N, K, lda, ldb


def time_variants(libs: dict[str, str], shapes: list[str], rounds: int = 5) -> list[dict]:
    """Interleaved timing of each library's sgemm on each shape (see module doc)."""
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("timing variants needs a GPU")
    vp, i = ctypes.c_void_p, ctypes.c_int
    loaded = {}
    for name, path in libs.items():
        lib = ctypes.CDLL(os.path.abspath(path))
        lib.sgemm.argtypes = [i, i, i, vp, i, vp, i, vp, i, vp, i]
        lib.sgemm.restype = i
        loaded[name] = lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    variant_mfma = 3  # SGEMM_MFMA

    def run(lib, A, B, C, reps):
        M, K = A.shape
        N = B.shape[1]
        for _ in range(reps):
            rc = lib.sgemm(M, N, K, A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0), C.data_ptr(),
                           C.stride(0), stream, variant_mfma)
            if rc != 0:
                raise RuntimeError(f"sgemm returned {rc}")

    # About 60 ms of 4096^3 products bring the chip to its sustained clock.
    X = torch.rand(4096, 4096, device=dev)
    Y = torch.empty_like(X)
    run(next(iter(loaded.values())), X, X, Y, 60)
    torch.cuda.synchronize()
    del X, Y
    results = []
    for spec in shapes:
        M, N, K, lda, ldb = _parse_shape(spec)
        g = torch.Generator(device=dev).manual_seed(M * 7 + N * 3 + K)
        A = torch.rand(M, lda, device=dev, generator=g)[:, :K]
        B = torch.rand(K, ldb, device=dev, generator=g)[:, :N]
        ref = A.double() @ B.double()
        bound = K * 2.0 ** -24 * (A.double().abs() @ B.double().abs()) + 1e-30
        entry = {"shape": spec, "variants": {}}
        for name, lib in loaded.items():
            C = torch.full((M, N), float("nan"), device=dev)
            run(lib, A, B, C, 1)
            torch.cuda.synchronize()
            worst = ((C.double() - ref).abs() / bound).max().item()
            if not worst < 1.0:
                raise RuntimeError(f"{name} on {spec}: error {worst} of the bound")
            entry["variants"][name] = {"worst_over_bound": worst, "us": []}
        del ref, bound
        C = torch.empty(M, N, device=dev)
        reps = min(2000, max(20, int(3e12 / (2.0 * M * N * K))))
        for _ in range(rounds):
            for name, lib in loaded.items():
                run(lib, A, B, C, 10)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                run(lib, A, B, C, reps)
                e1.record()
                e1.synchronize()
                entry["variants"][name]["us"].append(e0.elapsed_time(e1) * 1e3 / reps)
        line = f"{spec}:"
        for name, v in entry["variants"].items():
            us = sorted(v["us"])[len(v["us"]) // 2]
            v["median_us"] = us
            v["tflops"] = 2.0 * M * N * K / us / 1e6
            line += f"  {name} {us:9.2f} us {v['tflops']:6.1f} TF (err/bound {v['worst_over_bound']:.4f})"
        print(line, flush=True)
        results.append(entry)
    return results


def main(argv: list[str]) -> int:
    if len(argv) >= 2 and argv[0] == "build":
        print(build_variant(argv[1], argv[2:]))
        return 0
    if len(argv) == 3 and argv[0] == "time":
        libs = dict(spec.split("=", 1) for spec in argv[1].split(","))
        time_variants(libs, argv[2].split(","))
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
