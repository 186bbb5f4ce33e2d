"""Pins of the oracle's gradients (CPU).

The forward is linear in x and in the weights, so the gradients with respect
to them are fixed exactly by directional identities: for any direction d,
sum(grad_out * forward(x = d)) = sum(grad_x * d), and likewise for the
weights.  The offsets enter through the bilinear kernel, pinned by central
finite differences of the double-precision forward away from the kinks
(integer coordinates and the image border), where it is smooth.
"""
import numpy as np
import pytest

from oracle import ref
from tests import helpers as H


def case(rng, N=1, Hh=5, Ww=6, G=2, Cg=3, K=3, stride=1, pad=1, dil=1, std=1.5, rc=False):
    P = K * K - (1 if rc else 0)
    Ho = ref.output_dim(Hh, K, stride, pad, dil)
    Wo = ref.output_dim(Ww, K, stride, pad, dil)
    x = rng.standard_normal((N, Hh, Ww, G * Cg))
    off = rng.standard_normal((N, Ho, Wo, G * 2 * P)) * std
    m = rng.standard_normal((N, Ho, Wo, G * P))
    go = rng.standard_normal((N, Ho, Wo, G * Cg))
    kw = dict(K=K, stride=stride, pad=pad, dil=dil, remove_center=rc)
    return x, off, m, go, kw


GEOMS = [dict(), dict(K=3, stride=2, pad=0), dict(K=3, dil=2, pad=2), dict(K=5, pad=2), dict(K=1, pad=0),
         dict(rc=True), dict(G=1, Cg=5)]


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: ",".join(f"{k}={v}" for k, v in g.items()) or "default")
def test_grad_x_directional_identity(geom):
    rng = np.random.default_rng(31)
    x, off, m, go, kw = case(rng, **geom)
    gx, _, _ = ref.backward_f64(x, off, m, go, **kw)
    for _ in range(3):
        d = rng.standard_normal(x.shape)
        lhs = np.sum(go * ref.forward_f64(d, off, m, **kw))
        assert abs(lhs - np.sum(gx * d)) <= 1e-11 * (1 + abs(lhs))


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: ",".join(f"{k}={v}" for k, v in g.items()) or "default")
def test_grad_mask_directional_identity(geom):
    rng = np.random.default_rng(32)
    x, off, m, go, kw = case(rng, **geom)
    _, _, gm = ref.backward_f64(x, off, m, go, **kw)
    for _ in range(3):
        d = rng.standard_normal(m.shape)
        lhs = np.sum(go * ref.forward_f64(x, off, d, **kw))
        assert abs(lhs - np.sum(gm * d)) <= 1e-11 * (1 + abs(lhs))


def _smooth_offsets(rng, off, kw, Hh, Ww, scale=1.0, margin=1e-3):
    """Move each offset so that its sampling position is at least `margin`
    away from an integer and from the border band edges."""
    N, Ho, Wo, R = off.shape
    K, s, p, d = kw["K"], kw["stride"], kw["pad"], kw["dil"]
    P = K * K - (1 if kw["remove_center"] else 0)
    G = R // (2 * P)
    pts = [(i, j) for i in range(K) for j in range(K) if not (kw["remove_center"] and i == K // 2 and j == K // 2)]
    out = off.copy()
    for n, ho, wo, g, k, pl in np.ndindex(N, Ho, Wo, G, P, 2):
        i, j = pts[k]
        base = (wo * s - p + j * d) if pl == 0 else (ho * s - p + i * d)
        idx = (n, ho, wo, g * 2 * P + pl * P + k)
        pos = base + scale * out[idx]
        frac = pos - np.floor(pos)
        if frac < margin:
            pos += margin
        elif frac > 1 - margin:
            pos -= margin
        out[idx] = (pos - base) / scale
    return out


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: ",".join(f"{k}={v}" for k, v in g.items()) or "default")
def test_grad_offset_finite_differences(geom):
    rng = np.random.default_rng(33)
    x, off, m, go, kw = case(rng, **geom)
    scale = 0.75
    off = _smooth_offsets(rng, off, kw, x.shape[1], x.shape[2], scale=scale)
    _, goff, _ = ref.backward_f64(x, off, m, go, offset_scale=scale, **kw)
    h = 1e-7
    num = np.zeros_like(off)
    for idx in np.ndindex(off.shape):
        a, b = off.copy(), off.copy()
        a[idx] += h
        b[idx] -= h
        num[idx] = (np.sum(go * ref.forward_f64(x, a, m, offset_scale=scale, **kw)) -
                    np.sum(go * ref.forward_f64(x, b, m, offset_scale=scale, **kw))) / (2 * h)
    assert np.max(np.abs(num - goff)) <= 1e-6 * (1 + np.max(np.abs(goff)))


def test_points_outside_have_zero_gradient():
    rng = np.random.default_rng(34)
    x, off, m, go, kw = case(rng)
    for fill in (50.0, -50.0, np.nan):
        o = np.full_like(off, fill)
        gx, goff, gm = ref.backward_f64(x, o, m, go, **kw)
        assert not np.any(gx) and not np.any(goff) and not np.any(gm)


def test_offset_scale_chain_rule():
    """Same sampling positions from offsets o/s at scale s: the offset
    gradient is s times the one at scale 1."""
    rng = np.random.default_rng(35)
    x, off, m, go, kw = case(rng)
    g1 = ref.backward_f64(x, off, m, go, offset_scale=1.0, **kw)
    g3 = ref.backward_f64(x, off / 4.0, m, go, offset_scale=4.0, **kw)
    np.testing.assert_allclose(g3[0], g1[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g3[1], 4.0 * g1[1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g3[2], g1[2], rtol=1e-12, atol=1e-12)


def test_integer_offsets_gather_transpose():
    """Integer offsets and K=1: out = m * x[p + d]; grad_x scatters m * g to
    p + d exactly, grad_mask = g . x[p + d]; the offset gradient is the
    forward difference x[p + d + 1] - x[p + d] (derivative from the right)."""
    rng = np.random.default_rng(36)
    N, Hh, Ww, C = 1, 6, 7, 4
    x = rng.standard_normal((N, Hh, Ww, C))
    off = rng.integers(-1, 2, size=(N, Hh, Ww, 2)).astype(np.float64)
    m = rng.standard_normal((N, Hh, Ww, 1))
    go = rng.standard_normal((N, Hh, Ww, C))
    gx, goff, gm = ref.backward_f64(x, off, m, go, K=1, pad=0)
    want_x = np.zeros_like(x)
    want_m = np.zeros_like(m)
    want_o = np.zeros_like(off)
    xp = np.zeros((Hh + 1, Ww + 1, C))
    xp[:Hh, :Ww] = x[0]
    for r in range(Hh):
        for q in range(Ww):
            qy, qx = r + int(off[0, r, q, 1]), q + int(off[0, r, q, 0])
            if 0 <= qy < Hh and 0 <= qx < Ww:
                want_x[0, qy, qx] += m[0, r, q, 0] * go[0, r, q]
                want_m[0, r, q, 0] = np.dot(go[0, r, q], x[0, qy, qx])
                want_o[0, r, q, 0] = m[0, r, q, 0] * np.dot(go[0, r, q], xp[qy, qx + 1] - x[0, qy, qx])
                want_o[0, r, q, 1] = m[0, r, q, 0] * np.dot(go[0, r, q], xp[qy + 1, qx] - x[0, qy, qx])
    np.testing.assert_allclose(gx, want_x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gm, want_m, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(goff, want_o, rtol=1e-13, atol=1e-13)


def test_bounds_dominate_the_gradients():
    rng = np.random.default_rng(37)
    x, off, m, go, kw = case(rng, Hh=7, Ww=8)
    gx, goff, gm, b = ref.backward_f64(x, off, m, go, bounds=True, **kw)
    assert np.all(np.abs(gx) <= b["abs_x"] * (1 + 1e-12))
    assert np.all(np.abs(gm) <= b["abs_mask"] * (1 + 1e-12))
    assert np.all(np.abs(goff) <= 2 * b["abs_offset"] * (1 + 1e-12))
    assert np.array_equal(b["cnt_x"], np.round(b["cnt_x"])) and b["cnt_x"].max() >= 1


def _nonnegative_case(rng, Hh=7, Ww=8, G=2, Cg=3, std=2.0, **geom):
    """x, grad_out and weights >= 0 (weights on both sides of 1): every term
    of grad_x and grad_mask is then >= 0."""
    x, off, m, go, kw = case(rng, Hh=Hh, Ww=Ww, G=G, Cg=Cg, std=std, **geom)
    return np.abs(x), off, 2.0 * np.abs(m), np.abs(go), kw


def _positions(off, kw, Hh, Ww, scale):
    """(pts, px, py): sampling positions of every (n, ho, wo, g, k) in float64,
    p = base + scale * offset, with pts the (i, j) of point k."""
    N, Ho, Wo, R = off.shape
    K, s, p, d = kw["K"], kw["stride"], kw["pad"], kw["dil"]
    pts = [(i, j) for i in range(K) for j in range(K) if not (kw["remove_center"] and i == K // 2 and j == K // 2)]
    P = len(pts)
    G = R // (2 * P)
    o = off.reshape(N, Ho, Wo, G, 2, P)
    ii = np.array([i for i, _ in pts], dtype=np.float64)
    jj = np.array([j for _, j in pts], dtype=np.float64)
    bx = (np.arange(Wo) * s - p)[None, None, :, None, None] + jj * d
    by = (np.arange(Ho) * s - p)[None, :, None, None, None] + ii * d
    return pts, bx + scale * o[..., 0, :], by + scale * o[..., 1, :]


def _in_range(px, py, Hh, Ww):
    return (px > -1) & (px < Ww) & (py > -1) & (py < Hh)


GEOMS_B = [dict(), dict(K=3, stride=2, pad=0), dict(K=5, pad=2, dil=2), dict(rc=True)]


@pytest.mark.parametrize("geom", GEOMS_B, ids=lambda g: ",".join(f"{k}={v}" for k, v in g.items()) or "default")
def test_bound_sums_equal_the_gradients_when_every_term_is_nonnegative(geom):
    """With x, grad_out and the weights >= 0 every term of grad_x and
    grad_mask is >= 0, so their absolute-value sums are the gradients
    themselves, exactly (same terms, same order).  A bound sum with a term
    too many, a factor missing or a wrong corner differs."""
    rng = np.random.default_rng(39)
    x, off, m, go, kw = _nonnegative_case(rng, **geom)
    gx, goff, gm, b = ref.backward_f64(x, off, m, go, bounds=True, **kw)
    assert np.array_equal(b["abs_x"], gx) and gx.max() > 0
    assert np.array_equal(b["abs_mask"], gm) and gm.max() > 0


@pytest.mark.parametrize("geom", GEOMS_B, ids=lambda g: ",".join(f"{k}={v}" for k, v in g.items()) or "default")
def test_term_counts_equal_a_brute_force_count(geom):
    """cnt_x[q, c] = the number of (unit, point) pairs of c's group whose
    sampling position is in range and within the triangle kernel's support
    of pixel q (|py - qy| < 1 and |px - qx| < 1), counted by brute force over
    every pixel.  Random offsets: no position is an integer."""
    rng = np.random.default_rng(40)
    Hh, Ww, G, Cg = 7, 8, 2, 3
    x, off, m, go, kw = case(rng, Hh=Hh, Ww=Ww, G=G, Cg=Cg, std=2.0, **geom)
    _, _, _, b = ref.backward_f64(x, off, m, go, bounds=True, **kw)
    _, px, py = _positions(off, kw, Hh, Ww, 1.0)
    want = np.zeros((x.shape[0], Hh, Ww, G))
    qy = np.arange(Hh)[:, None]
    qx = np.arange(Ww)[None, :]
    for idx in np.ndindex(px.shape):
        n, _, _, g, _ = idx
        if not _in_range(px[idx], py[idx], Hh, Ww):
            continue
        want[n, :, :, g] += (np.abs(py[idx] - qy) < 1) & (np.abs(px[idx] - qx) < 1)
    assert np.array_equal(b["cnt_x"], np.repeat(want, Cg, axis=-1))


@pytest.mark.parametrize("geom", GEOMS_B, ids=lambda g: ",".join(f"{k}={v}" for k, v in g.items()) or "default")
def test_offset_bound_sums_equal_a_brute_force_triangle_kernel_sum(geom):
    """abs_offset of point k, plane x: |scale * m_k| times the sum over
    channels c and every pixel q of |g_c| * tri(py - qy) * |dtri(px - qx)| *
    |x[q, c]| (the absolute terms of d sample / d px in triangle-kernel form,
    dtri = -1 on [0, 1) and +1 on [-1, 0)); plane y with the roles of the
    axes exchanged.  Brute force over all pixels."""
    rng = np.random.default_rng(41)
    Hh, Ww, G, Cg = 6, 7, 2, 3
    scale = 0.75
    x, off, m, go, kw = case(rng, Hh=Hh, Ww=Ww, G=G, Cg=Cg, std=2.0, **geom)
    _, _, _, b = ref.backward_f64(x, off, m, go, bounds=True, offset_scale=scale, **kw)
    pts, px, py = _positions(off, kw, Hh, Ww, scale)
    P = len(pts)
    N, Ho, Wo, _ = off.shape
    tri = lambda t: np.maximum(0.0, 1.0 - np.abs(t))  # noqa: E731
    dtri_abs = lambda t: ((t >= -1) & (t < 1)).astype(np.float64)  # noqa: E731
    want = np.zeros((N, Ho, Wo, G, 2, P))
    qy = np.arange(Hh)[:, None]
    qx = np.arange(Ww)[None, :]
    mm = m.reshape(N, Ho, Wo, G, P)
    for n, ho, wo, g, k in np.ndindex(N, Ho, Wo, G, P):
        X, Y = px[n, ho, wo, g, k], py[n, ho, wo, g, k]
        if not _in_range(X, Y, Hh, Ww):
            continue
        ax = np.abs(go[n, ho, wo, g * Cg:(g + 1) * Cg])           # |g_c|
        f = np.abs(x[n, :, :, g * Cg:(g + 1) * Cg])               # |x[q, c]|
        wx = (tri(Y - qy) * dtri_abs(X - qx))[..., None]
        wy = (dtri_abs(Y - qy) * tri(X - qx))[..., None]
        sm = abs(scale * mm[n, ho, wo, g, k])
        want[n, ho, wo, g, 0, k] = sm * np.sum(wx * f * ax)
        want[n, ho, wo, g, 1, k] = sm * np.sum(wy * f * ax)
    np.testing.assert_allclose(b["abs_offset"], want.reshape(off.shape), rtol=1e-12, atol=0)


def test_f32_positions_equal_exact_positions_for_dyadic_offsets():
    """Offsets that are multiples of 1/64 (and scale 0.5) give positions that
    binary32 represents exactly: both position modes agree exactly; with
    general offsets they differ only through the rounding of the positions."""
    rng = np.random.default_rng(38)
    x, off, m, go, kw = case(rng)
    dy = np.round(off * 64) / 64
    a = ref.backward_f64(x, dy, m, go, offset_scale=0.5, **kw)
    b = ref.backward_f64(x, dy, m, go, offset_scale=0.5, f32_positions=True, **kw)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    c = ref.backward_f64(x, off, m, go, offset_scale=0.3, **kw)
    d = ref.backward_f64(x, off, m, go, offset_scale=0.3, f32_positions=True, **kw)
    assert not all(np.array_equal(u, v) for u, v in zip(c, d))
    for u, v in zip(c, d):
        np.testing.assert_allclose(u, v, rtol=1e-4, atol=1e-4)
