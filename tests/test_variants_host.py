"""Host logic of the variant build and timing tool (no GPU, no full build)."""

import pytest
import torch

from dense_fp32_matrix_sgemm_amd import _build, variants


def test_parse_shape():
    assert variants._parse_shape("1024x1024x1024") == (1024, 1024, 1024, 1024, 1024)
    assert variants._parse_shape("3001x2047x4093:4100:2050") == (3001, 2047, 4093, 4100, 2050)
    for bad in ("0x4x4", "4x4x4:3", "4x4x4:4:3"):
        with pytest.raises(ValueError):
            variants._parse_shape(bad)


def test_failed_build_restores_settings(tmp_path):
    before = (list(_build.HIPCC_FLAGS), _build.OBJDIR, _build.LIBDIR, _build.LIB_PATH)
    with pytest.raises(RuntimeError):
        variants.build_variant(str(tmp_path / "v"), ["-include", str(tmp_path / "missing.h")])
    assert (_build.HIPCC_FLAGS, _build.OBJDIR, _build.LIBDIR, _build.LIB_PATH) == before


def test_usage_and_no_gpu(capsys):
    assert variants.main([]) == 2
    if not torch.cuda.is_available():
        with pytest.raises(RuntimeError):
            variants.time_variants({}, ["8x8x8"])
