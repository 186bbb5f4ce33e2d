"""Pins of the module oracle (oracle/module.py), as functions of the module
object so that the same checks can run against planted-mistake copies.
Each pin compares with a library routine (torch float64 on the CPU), a
closed form or an invariant; none retypes the oracle's own expression."""
import numpy as np
import torch
import torch.nn.functional as F


def _nchw(a):
    return torch.from_numpy(np.ascontiguousarray(a.transpose(0, 3, 1, 2)))


def _nhwc(t):
    return t.numpy().transpose(0, 2, 3, 1)


def pin_conv1x1(mod):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 5, 6, 7))
    w = rng.standard_normal((9, 7))
    b = rng.standard_normal(9)
    want = _nhwc(F.conv2d(_nchw(x), torch.from_numpy(w)[:, :, None, None], torch.from_numpy(b)))
    np.testing.assert_allclose(mod.conv1x1(x, w, b), want, rtol=1e-12, atol=1e-12)
    # a square matrix, so that a transposed weight would not fail on shape
    w2 = rng.standard_normal((7, 7))
    want2 = _nhwc(F.conv2d(_nchw(x), torch.from_numpy(w2)[:, :, None, None]))
    np.testing.assert_allclose(mod.conv1x1(x, w2, np.zeros(7)), want2, rtol=1e-12, atol=1e-12)


def pin_group_norm(mod):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 4, 5, 12)) * 3 + 1.5
    gamma, beta = rng.standard_normal(12), rng.standard_normal(12)
    for groups in (1, 3, 12):
        want = _nhwc(F.group_norm(_nchw(x), groups, torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-5))
        np.testing.assert_allclose(mod.group_norm(x, groups, gamma, beta, 1e-5), want, rtol=1e-11, atol=1e-11)
    # a constant group normalises to beta exactly
    c = np.full((1, 3, 3, 4), 2.5)
    np.testing.assert_array_equal(mod.group_norm(c, 2, np.ones(4), beta[:4], 1e-5), np.broadcast_to(beta[:4], c.shape))


def pin_layer_norm(mod):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 4, 5, 10)) * 2 - 0.7
    gamma, beta = rng.standard_normal(10), rng.standard_normal(10)
    want = F.layer_norm(torch.from_numpy(x), (10,), torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-6)
    np.testing.assert_allclose(mod.layer_norm(x, gamma, beta, 1e-6), want.numpy(), rtol=1e-11, atol=1e-11)


def pin_dwconv3x3(mod):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 5, 7, 6))
    w = rng.standard_normal((6, 3, 3))
    b = rng.standard_normal(6)
    want = _nhwc(F.conv2d(_nchw(x), torch.from_numpy(w)[:, None], torch.from_numpy(b), padding=1, groups=6))
    np.testing.assert_allclose(mod.dwconv3x3(x, w, b), want, rtol=1e-12, atol=1e-12)
    # a one-hot tap shifts the image: w[c, 0, 2] picks x[h - 1, w + 1]
    e = np.zeros((6, 3, 3))
    e[:, 0, 2] = 1.0
    got = mod.dwconv3x3(x, e, np.zeros(6))
    np.testing.assert_array_equal(got[:, 1:, :-1], x[:, :-1, 1:])
    np.testing.assert_array_equal(got[:, 0], 0.0)


def pin_centre_scale(mod):
    rng = np.random.default_rng(5)
    y = rng.standard_normal((1, 3, 4, 8))
    xc = rng.standard_normal((1, 3, 4, 8))
    # logit 0: the gate is 1/2, the mean of the two features
    np.testing.assert_allclose(mod.centre_scale(y, xc, np.zeros((1, 3, 4, 2)), 2), (y + xc) / 2, rtol=1e-15)
    # saturated gates select one feature, per group
    lg = np.zeros((1, 3, 4, 2))
    lg[..., 0], lg[..., 1] = 800.0, -800.0
    got = mod.centre_scale(y, xc, lg, 2)
    np.testing.assert_array_equal(got[..., :4], xc[..., :4])
    np.testing.assert_array_equal(got[..., 4:], y[..., 4:])
    t = rng.standard_normal(20) * 4
    np.testing.assert_allclose(mod.sigmoid(t), torch.sigmoid(torch.from_numpy(t)).numpy(), rtol=1e-14)


def pin_split_params(mod):
    G, P = 3, 9
    rows = np.arange(2 * 3 * 3 * G * P, dtype=np.float64).reshape(2, 1, 3, 3 * G * P)
    off, m = mod.split_params(rows, G, P)
    assert off.shape[-1] == 2 * G * P and m.shape[-1] == G * P
    # group g's x-offset of point k is channel g*2P + k, its y-offset g*2P + P + k,
    # its weight 2*G*P + g*P + k (the listing's reshape to (G, 2, K*K) and (G, K*K))
    assert off[0, 0, 0, 1 * 2 * P + 4] == rows[0, 0, 0, 2 * P + 4]
    assert m[0, 0, 0, 2 * P + 3] == rows[0, 0, 0, 2 * G * P + 2 * P + 3]


def pin_abs_terms(mod):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 3, 3, 5))
    w, b = rng.standard_normal((4, 5)), rng.standard_normal(4)
    np.testing.assert_allclose(mod.abs_terms_conv1x1(x, w, b),
                               mod.conv1x1(np.abs(x), np.abs(w), np.abs(b)), rtol=1e-15)
    # non-negative operands: the bound sum is the value itself
    xa, wa, ba = np.abs(x), np.abs(w), np.abs(b)
    np.testing.assert_allclose(mod.abs_terms_conv1x1(xa, wa, ba), mod.conv1x1(xa, wa, ba), rtol=1e-15)
    wd = np.abs(rng.standard_normal((5, 3, 3)))
    np.testing.assert_allclose(mod.abs_terms_dwconv3x3(xa, wd, ba[:1].repeat(5)),
                               mod.dwconv3x3(xa, wd, ba[:1].repeat(5)), rtol=1e-15)


PINS = [pin_conv1x1, pin_group_norm, pin_layer_norm, pin_dwconv3x3, pin_centre_scale, pin_split_params,
        pin_abs_terms]
