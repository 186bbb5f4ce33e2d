"""The seeded generator (CPU only)."""
import math

import numpy as np
import pytest

from deformable_convolution_vision_dcnv4_amd import inputs as gen
from deformable_convolution_vision_dcnv4_amd.workloads import SENSITIVITY, WORKLOADS


def test_splitmix_known_values():
    # splitmix64 with state 0 yields 0xE220A8397B1DCDAF first (published test vector
    # of the reference generator in Vigna's splitmix64.c); our word() with key=0
    # and counter 0 is mix(0 + 1*GOLDEN), the same first output.
    z = gen._mix(np.uint64(0) + gen.GOLDEN)
    assert int(z) == 0xE220A8397B1DCDAF


def test_counter_based_and_deterministic():
    a = gen.draw(0, 1, 10000, ("normal", 1.0))
    b = gen.draw(0, 1, 10000, ("normal", 1.0))
    assert np.array_equal(a, b)
    # element i does not depend on how many are drawn or on chunking
    c = gen.draw(0, 1, 5000, ("normal", 1.0))
    assert np.array_equal(a[:5000], c)
    u = gen.uniform_words(0, 2, 0, 1000)
    v = gen.uniform_words(0, 2, 500, 500)
    assert np.array_equal(u[500:], v)
    assert not np.array_equal(gen.draw(1, 1, 100, ("normal", 1.0)), a[:100])
    assert not np.array_equal(gen.draw(0, 2, 100, ("normal", 1.0)), a[:100])


@pytest.mark.parametrize("dist", [("normal", 1.0), ("normal", 3.0), ("uniform", -1.0, 1.0)])
def test_moments(dist):
    v = gen.draw(0, 0, 400000, dist)
    if dist[0] == "normal":
        assert abs(v.mean()) < 0.01 * dist[1]
        assert abs(v.std() - dist[1]) < 0.01 * dist[1]
        assert abs(np.mean(np.abs(v) < dist[1]) - 0.6827) < 0.005
    else:
        assert v.min() >= -1.0 and v.max() < 1.0
        assert abs(v.mean()) < 0.01 and abs(v.var() - 1.0 / 3.0) < 0.01


def test_io_rounding_is_nearest_even():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11])
    b = gen.to_io(v, "bf16")
    assert list(b) == [0x3F80, 0x3F82, 0x3F80, 0x3F80]
    h = gen.to_io(v, "f16").view(np.uint16)
    assert list(h) == [0x3C04, 0x3C0C, 0x3C00, 0x3C02]


def test_integer_offsets_and_shapes():
    wl = WORKLOADS["tiny"]
    x, off, m = gen.make_inputs(wl, "f32", integer_offsets=True)
    assert x.shape == (1, 16, 16, 64) and off.shape == (1, 16, 16, 72) and m.shape == (1, 16, 16, 36)
    assert np.array_equal(off, np.rint(off))
    x2, off2, m2 = gen.make_inputs(wl, "f32")
    assert np.array_equal(x, x2) and np.array_equal(m, m2)
    assert not np.array_equal(off, off2)


def test_workload_byte_counts():
    # algorithmic bytes: x once + out once + 3*P offsets/weights per (pixel, group)
    assert WORKLOADS["tiny"].algorithmic_bytes("f32") == 241664
    assert WORKLOADS["fiit_stage1"].algorithmic_bytes("f32") == 189464576
    assert WORKLOADS["fiit_stage1"].algorithmic_bytes("f16") == 94732288
    assert WORKLOADS["fiit_stage3"].algorithmic_bytes("f16") == 23683072
    assert WORKLOADS["hires"].algorithmic_bytes("bf16") == 123731968
    assert WORKLOADS["sd_latent"].algorithmic_bytes("bf16") == 56098816
    assert WORKLOADS["sd_latent"].mask_dist[1] == pytest.approx(1 / math.sqrt(8))


def test_smooth_offsets_keep_the_distribution_and_correlate_neighbours():
    """Box-filtered offsets (radius 2, divided by 5): still N(0, sigma) per
    element, while horizontally adjacent pixels share 20 of their 25 terms
    (correlation 4/5); the other tensors and the offsets' draws are those
    of the unsmoothed workload."""
    import dataclasses
    wl = dataclasses.replace(SENSITIVITY["fiit_stage1_smooth"], N=4)
    base = dataclasses.replace(wl, offset_smooth=0)
    x, off, m = gen.make_inputs(wl, "f32")
    x0, off0, m0 = gen.make_inputs(base, "f32")
    assert np.array_equal(x, x0) and np.array_equal(m, m0)
    o = off.astype(np.float64)
    assert abs(o.std() / 1.5 - 1.0) < 0.02 and abs(o.mean()) < 0.02
    a, b = o[:, :, :-1, :].ravel(), o[:, :, 1:, :].ravel()
    assert abs(np.corrcoef(a, b)[0, 1] - 0.8) < 0.02
    # the box sum written out for one element, against the vectorised form
    raw = gen.draw(wl.seed, gen.STREAM_OFFSET, off0.size, wl.offset_dist).reshape(off0.shape)
    n, y, xx, c = 1, 0, 55, 7
    s = sum(raw[n, (y + dy) % 56, (xx + dx) % 56, c] for dy in range(-2, 3) for dx in range(-2, 3)) / 5
    assert np.float32(s) == off[n, y, xx, c]
    # radius 0 is the identity
    assert np.array_equal(gen.box_smooth(raw, 0), raw)
