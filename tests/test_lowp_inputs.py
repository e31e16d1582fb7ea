"""The reduced-precision workload's inputs and their exact widening (host).

The path multiplies bf16 or f16 operands with FP32 accumulation (the pages'
tensor-core variant, "Matrix Multiplication -- Naive to Tiled", section 07,
with FP32 accumulation). Every 16-bit value widens to float32 exactly, so the
oracle of this workload is the pinned general-form oracle applied to the
widened operands; what needs pinning here is the widening itself and the
generator's grids.
"""

import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.mark.parametrize("bits,value", [(0x3F80, 1.0), (0xC000, -2.0), (0x3E80, 0.25), (0x0000, 0.0),
                                        (0x4049, 3.140625), (0x7F7F, 3.3895313892515355e38),
                                        (0x0001, 2.0**-133), (0x7F80, np.inf), (0xFF80, -np.inf)])
def test_bf16_known_encodings(bits, value):
    assert oracle.lowp_to_float32(np.array([bits], np.uint16), "bf16")[0] == np.float32(value)


@pytest.mark.parametrize("bits,value", [(0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0001, 2.0**-24),
                                        (0x0400, 2.0**-14), (0x03FF, 1023 * 2.0**-24), (0x3555, 0.333251953125),
                                        (0x7C00, np.inf), (0xFC00, -np.inf), (0x8000, -0.0)])
def test_f16_known_encodings(bits, value):
    got = oracle.lowp_to_float32(np.array([bits], np.uint16), "f16")[0]
    assert got == np.float32(value) and np.signbit(got) == np.signbit(np.float32(value))


def test_every_encoding_matches_library_conversions():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    # f16: numpy's binary16 conversion; NaN payloads aside, every code agrees.
    ours = oracle.lowp_to_float32(codes, "f16")
    ref = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # bf16: torch's bfloat16 conversion.
    ours = oracle.lowp_to_float32(codes, "bf16")
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dist", ["u01", "pm1", "int"])
def test_generator_values_round_trip_exactly(dtype, dist):
    x = synth.lowp_values(7, (300, 257), dtype, dist)
    bits = synth.to_lowp_bits(x, dtype)
    assert bits.dtype == np.uint16
    assert np.array_equal(oracle.lowp_to_float32(bits, dtype), x)
    lo, hi = (-1.0, 1.0) if dist == "pm1" else (0.0, 1.0)
    if dist != "int":
        assert x.min() >= lo and x.max() < hi
        step = 2.0 ** -(synth.LOWP_BITS[dtype] - (1 if dist == "pm1" else 0))
        assert np.array_equal(x / step, np.round(x / step))      # on the stated grid
        assert len(np.unique(x)) > 100                          # and not degenerate


def test_generator_rejects_inexact_values():
    with pytest.raises(ValueError):
        synth.to_lowp_bits(np.array([1.0 + 2.0**-10], np.float32), "bf16")
    with pytest.raises(ValueError):
        synth.to_lowp_bits(np.array([1.0 + 2.0**-12], np.float32), "f16")
