"""Pins of the seeded input generator (host only)."""

import numpy as np
import pytest

import synth


def test_splitmix64_published_sequence():
    # Outputs of the sequential SplitMix64 generator from state 1234567, as
    # printed with the published reference implementation.
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [synth.splitmix64_scalar(1234567, i) for i in range(5)] == want
    assert [int(v) for v in synth.splitmix64(1234567, 5)] == want


def test_splitmix64_seed_zero_first_output():
    assert synth.splitmix64_scalar(0, 0) == 0xE220A8397B1DCDAF


def test_vector_form_matches_scalar_definition():
    for seed in (0, 42, 43, 2**64 - 1):
        v = synth.splitmix64(seed, 50, offset=1000)
        assert [int(x) for x in v] == [synth.splitmix64_scalar(seed, 1000 + i)
                                       for i in range(50)]


def test_uniform01_grid_and_range():
    x = synth.uniform01(42, (300, 301))
    assert x.dtype == np.float32
    assert x.min() >= 0.0 and x.max() < 1.0
    scaled = x.astype(np.float64) * 2**24
    assert np.array_equal(scaled, np.round(scaled))       # on the 2^-24 grid
    assert abs(float(x.mean()) - 0.5) < 0.01


def test_uniform_pm1_grid_and_range():
    x = synth.uniform_pm1(43, (300, 301))
    assert x.min() >= -1.0 and x.max() < 1.0
    scaled = x.astype(np.float64) * 2**23
    assert np.array_equal(scaled, np.round(scaled))
    assert abs(float(x.mean())) < 0.01
    assert (x < 0).any() and (x > 0).any()


def test_small_int_range():
    x = synth.small_int(7, (100, 100))
    assert set(np.unique(x).tolist()) == set(range(-8, 9))


def test_reproducible_and_seed_sensitive():
    assert np.array_equal(synth.uniform01(42, (64, 64)), synth.uniform01(42, (64, 64)))
    assert not np.array_equal(synth.uniform01(42, (64, 64)), synth.uniform01(43, (64, 64)))


def test_embed_pads_with_fill():
    x = synth.uniform01(1, (5, 7))
    buf = synth.embed(x, 11)
    assert buf.shape == (5, 11)
    assert np.array_equal(buf[:, :7], x)
    assert np.isnan(buf[:, 7:]).all()
    with pytest.raises(ValueError):
        synth.embed(x, 6)


def test_integer_patterns_agree_on_host_and_device():
    # The two builders of a closed-form pattern give the same matrix (torch on
    # the CPU stands in for the device here), in block-sized pieces too, and
    # the values are the small integers the formula names.
    import torch
    for (rows, cols, mr, mc, mod, block) in [(1000, 40, 7, 13, 17, 300), (37, 4100, 5, 3, 11, 8), (5, 5, 1, 1, 3, 2)]:
        t = synth.pattern_device(rows, cols, mr, mc, mod, "cpu", block=block).numpy()
        h = synth.pattern_rows(np.arange(rows), cols, mr, mc, mod)
        assert np.array_equal(t, h)
        r, c = 3, 4
        assert h[r, c] == ((r * mr + c * mc) % mod) - mod // 2
        assert h.min() >= -(mod // 2) and h.max() <= mod - 1 - mod // 2
    b = synth.pattern_device(64, 64, 7, 13, 17, "cpu", dtype=torch.bfloat16)
    assert torch.equal(b.float(), synth.pattern_device(64, 64, 7, 13, 17, "cpu"))
