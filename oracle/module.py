"""Oracle of the DCNv4 module forward around the operator (test
infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline may use it; the product path never does).

Plain float64 numpy, one function per step, each written from the pages:

  jsqmd.com/news/933833 ("不只是卷积的平替：我把DCNv4塞进Stable Diffusion的
  U-Net里"), section 2, the DCNv4Block example and item 2 of the list before
  it: a 1x1 convolution adjusts the channels ("proj"), a normalisation
  follows ("norm"; the example writes GroupNorm(32, C), the list says
  LayerNorm, so both are offered), then ONE predictor produces offsets and
  dynamic weights together: a depthwise 3x3 convolution (padding 1) and a
  1x1 convolution to 3*G*9 channels, the first 2*G*9 being the offsets and
  the rest the weights, with no activation and no further normalisation
  between them.  The operator samples the normalised features.
  pwwt.cn/news/2159231 ("掌握DCNv4技术…"), section "进阶优化建议": centre
  feature scaling through a sigmoid, and removal of the centre point.

Readings where the pages are silent (stated in the design notes):
  - channels-last [N, H, W, C] throughout; a 1x1 convolution is a
    per-pixel product with a [C_out, C_in] matrix plus a bias;
  - group norm: per image and channel group, mean and biased variance over
    (H, W, channels of the group); layer norm: per pixel over C; both
    (v - mean) / sqrt(var + eps) * gamma + beta;
  - centre-feature scaling: a per-pixel, per-group gate
    s = sigmoid(xn . wc[g] + bc[g]) blends the aggregated feature with the
    pixel's own (centre) normalised feature: y * (1 - s) + xn * s;
  - an optional output projection (a 1x1 convolution) closes the module;
  - in a 16-bit run every step's output is rounded once to the I/O type
    before the next step reads it (``rnd``), as a framework running the
    steps one by one would store them.
"""
import numpy as np


def conv1x1(x, w, b):
    """x [..., Cin], w [Cout, Cin], b [Cout] -> [..., Cout]: per pixel w @ x + b."""
    return np.matmul(x, w.T) + b


def group_norm(x, groups, gamma, beta, eps):
    """x [N, H, W, C]: mean and biased variance per (image, channel group)."""
    N, H, W, C = x.shape
    v = x.reshape(N, H * W, groups, C // groups)
    mean = v.mean(axis=(1, 3), keepdims=True)
    var = ((v - mean) ** 2).mean(axis=(1, 3), keepdims=True)
    y = (v - mean) / np.sqrt(var + eps)
    return y.reshape(N, H, W, C) * gamma + beta


def layer_norm(x, gamma, beta, eps):
    """x [..., C]: mean and biased variance per pixel over the channels."""
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def dwconv3x3(x, w, b):
    """Depthwise 3x3 convolution, zero padding 1, stride 1: x [N, H, W, C],
    w [C, 3, 3] (w[c, i, j] multiplies x[h + i - 1, w + j - 1, c]), b [C]."""
    N, H, W, C = x.shape
    xp = np.zeros((N, H + 2, W + 2, C))
    xp[:, 1:H + 1, 1:W + 1] = x
    out = np.zeros((N, H, W, C)) + b
    for i in range(3):
        for j in range(3):
            out += xp[:, i:i + H, j:j + W, :] * w[:, i, j]
    return out


def sigmoid(t):
    return 1.0 / (1.0 + np.exp(-t))


def centre_scale(y, xc, logits, G):
    """y, xc [N, H, W, G*Cg]; logits [N, H, W, G]: y * (1 - s) + xc * s with
    s = sigmoid(logits) for every channel of group g."""
    N, H, W, C = y.shape
    s = np.repeat(sigmoid(logits), C // G, axis=-1)
    return y * (1.0 - s) + xc * s


def abs_terms_conv1x1(x, w, b):
    """Sum of the absolute values of the terms of conv1x1 (error bounds)."""
    return np.matmul(np.abs(x), np.abs(w).T) + np.abs(b)


def abs_terms_dwconv3x3(x, w, b):
    return dwconv3x3(np.abs(x), np.abs(w), np.abs(b))


def split_params(rows, G, P):
    """The predictor's row [N, H, W, >= 3*G*P] as the operator reads it:
    offsets = the first 2*G*P channels, per group (x-offsets of the P
    points, then their y-offsets); weights = the next G*P channels, per
    group P raw weights."""
    return rows[..., :2 * G * P], rows[..., 2 * G * P:3 * G * P]
