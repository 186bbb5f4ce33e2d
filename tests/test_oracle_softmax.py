"""Pins of the DCNv3-style weight normalisation (CPU): a softmax over each
group's P points, per pixel (the step DCNv4 removes)."""
import numpy as np
import pytest
import scipy.special

from oracle import ref


@pytest.mark.parametrize("G,P", [(1, 9), (4, 9), (3, 8), (2, 25), (1, 1)])
def test_softmax_matches_library_routine(G, P):
    rng = np.random.default_rng(51)
    m = rng.standard_normal((2, 3, 4, G * P)) * 3
    got = ref.softmax_weights(m, groups=G, P=P)
    want = scipy.special.softmax(m.reshape(2, 3, 4, G, P), axis=-1).reshape(m.shape)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-16)


def test_softmax_rows_sum_to_one_positive_and_shift_invariant():
    rng = np.random.default_rng(52)
    G, P = 4, 9
    m = rng.standard_normal((1, 5, 6, G * P))
    w = ref.softmax_weights(m, groups=G, P=P)
    assert np.all(w > 0)
    np.testing.assert_allclose(w.reshape(1, 5, 6, G, P).sum(-1), 1.0, rtol=0, atol=1e-15)
    shift = np.repeat(rng.standard_normal((1, 5, 6, G)) * 50, P, axis=-1)
    np.testing.assert_allclose(ref.softmax_weights(m + shift, groups=G, P=P), w, rtol=1e-12, atol=1e-15)


def test_softmax_of_large_weights_does_not_overflow():
    m = np.array([[[[1000.0, 999.0, -1000.0, 1000.0]]]])
    w = ref.softmax_weights(m, groups=1, P=4)
    e = np.exp(np.array([0.0, -1.0, -2000.0, 0.0]))
    np.testing.assert_allclose(w[0, 0, 0], e / e.sum(), rtol=1e-15, atol=0)


def test_dcnv3_style_aggregation_is_dcnv4_with_normalised_weights():
    rng = np.random.default_rng(53)
    N, H, W, G, Cg, P = 1, 5, 6, 2, 3, 9
    x = rng.standard_normal((N, H, W, G * Cg))
    off = rng.standard_normal((N, H, W, G * 2 * P)) * 1.5
    m = rng.standard_normal((N, H, W, G * P))
    w = scipy.special.softmax(m.reshape(N, H, W, G, P), axis=-1).reshape(m.shape)
    np.testing.assert_allclose(ref.forward_softmax_f64(x, off, m), ref.forward_f64(x, off, w),
                               rtol=1e-13, atol=1e-13)
    # with zero offsets and equal weights it is the 3x3 box mean (zero padding)
    z = np.zeros_like(off)
    eq = np.zeros_like(m)
    xp = np.pad(x, ((0, 0), (1, 1), (1, 1), (0, 0)))
    box = sum(xp[:, i:i + H, j:j + W] for i in range(3) for j in range(3)) / 9.0
    np.testing.assert_allclose(ref.forward_softmax_f64(x, z, eq), box, rtol=1e-13, atol=1e-13)
