"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Every pin is chosen so that a plausible slip in the oracle -- a dropped
bilinear term, swapped offset planes, truncation instead of floor, a wrong
point order, a softmax left in, a sign error -- breaks at least one of them:

  formats      binary16 / bfloat16 decode and round-to-nearest-even encode
               against numpy and torch (library routines);
  brute force  the triangle-kernel sum over every pixel (tests/helpers.py);
  zero offsets grouped cross-correlation, torch.nn.functional.conv2d (float64);
  integer      exact shifted gathers on integer data (bit-exact);
  ramp         a linear image is reproduced exactly at fractional positions;
  half pixel   the mean of 2 and 4 neighbours;
  linearity    power-of-two and sign scaling of the weights (bit-exact);
  OOB          every point outside -> exact zero;
  groups       permuting groups permutes outputs;
  golden       hand-worked examples under tests/golden/.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import ref
from tests import helpers as H

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32(a):
    return np.asarray(a, dtype=np.float32)


def run32(x, off, m, **kw):
    return ref.forward_f32(f32(x), f32(off), f32(m), dtype="f32", **kw)


def run64(x, off, m, **kw):
    return ref.forward_f64(np.asarray(x, np.float64), np.asarray(off, np.float64),
                           np.asarray(m, np.float64), **kw)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_f16_decode_every_code():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = ref.to_f32(codes.view(np.float16), "f16")
    lib = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), lib[~nan].view(np.uint32))


def test_bf16_decode_every_code():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = ref.to_f32(codes, "bf16")
    lib = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), lib[~nan].view(np.uint32))


def _encode_probe(rng, mbits_small):
    """Random binary32 values spread over many binades, plus exact ties."""
    r = rng.standard_normal(200000) * np.exp2(rng.integers(-30, 20, 200000))
    vals = [r.astype(np.float32)]
    # exact midpoints between neighbours of the small format: low bits = 100..0
    bits = rng.integers(0, 1 << 31, 100000, dtype=np.uint64).astype(np.uint32)
    drop = 23 - mbits_small
    tie = (bits & ~np.uint32((1 << drop) - 1)) | np.uint32(1 << (drop - 1))
    vals.append(tie.view(np.float32))
    vals.append(np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.0, 65520.0, 65536.0,
                          2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -126,
                          2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -133, 3.4e38, -3.4e38],
                         dtype=np.float32))
    v = np.concatenate(vals)
    return v[np.isfinite(v) | np.isinf(v)]


def test_f16_encode_matches_numpy_rne():
    v = _encode_probe(np.random.default_rng(1), 10)
    mine = ref.from_f32(v, "f16").view(np.uint16)
    lib = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, lib)


def test_bf16_encode_matches_torch_rne():
    v = _encode_probe(np.random.default_rng(2), 7)
    mine = ref.from_f32(v, "bf16")
    lib = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, lib)


def test_encode_nan_stays_nan():
    v = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(np.isnan(ref.to_f32(ref.from_f32(v, "f16"), "f16")))
    assert np.all(np.isnan(ref.to_f32(ref.from_f32(v, "bf16"), "bf16")))


# --------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,K,s,p,d", [(16, 3, 1, 1, 1), (7, 3, 2, 0, 1), (5, 3, 1, 2, 2),
                                       (9, 5, 2, 1, 1), (1, 1, 1, 0, 1), (4, 3, 3, 1, 1)])
def test_output_dim_matches_conv2d(n, K, s, p, d):
    y = torch.nn.functional.conv2d(torch.zeros(1, 1, n, n), torch.zeros(1, 1, K, K),
                                   stride=s, padding=p, dilation=d)
    assert ref.output_dim(n, K, s, p, d) == y.shape[-1]


def test_output_dim_invalid_is_nonpositive():
    assert ref.output_dim(2, 5, 1, 0, 1) <= 0
    assert ref.output_dim(4, 3, 0, 1, 1) <= 0


# --------------------------------------------------------------------------
# brute force on tiny inputs
# --------------------------------------------------------------------------

BF_CASES = [
    # N H W G Cg K s p d scale rc
    (1, 5, 4, 1, 3, 3, 1, 1, 1, 1.0, False),
    (2, 4, 6, 2, 2, 3, 2, 1, 1, 1.0, False),
    (1, 6, 5, 3, 1, 3, 1, 2, 2, 0.5, False),
    (1, 3, 3, 2, 5, 1, 1, 0, 1, 2.0, False),
    (1, 7, 7, 1, 2, 2, 1, 0, 1, 1.0, False),
    (1, 1, 1, 1, 4, 3, 1, 1, 1, 1.0, False),
    (1, 5, 5, 2, 2, 3, 1, 1, 1, 1.0, True),
    (1, 2, 7, 1, 3, 3, 2, 2, 1, 1.0, False),
]


@pytest.mark.parametrize("case", BF_CASES)
@pytest.mark.parametrize("edges", [False, True])
def test_bruteforce_triangle_kernel(case, edges):
    N, Hh, Ww, G, Cg, K, s, p, d, scale, rc = case
    rng = np.random.default_rng(hash((case, edges)) % (1 << 32))
    x, off, m = H.random_case(rng, N, Hh, Ww, G, Cg, K, s, p, d, off_sigma=1.5, remove_center=rc)
    if edges:
        off = H.edge_offsets(rng, N, Hh, Ww, G, K, s, p, d, remove_center=rc) / scale
        off = off.astype(np.float32).astype(np.float64)
    kw = dict(K=K, stride=s, pad=p, dil=d, offset_scale=scale, remove_center=rc)
    bf = H.bruteforce_f64(x, off, m, K, s, p, d, scale=scale, remove_center=rc)
    o64 = run64(x, off, m, **kw)
    np.testing.assert_allclose(o64, bf, rtol=1e-12, atol=1e-12)
    o32 = run32(x, off, m, **kw).astype(np.float64)
    bound = H.f32_bound(x, off, m, K, s, p, d, scale=scale, remove_center=rc)
    assert np.all(np.abs(o32 - bf) <= bound + 1e-30), np.max(np.abs(o32 - bf) - bound)


# --------------------------------------------------------------------------
# zero offsets: grouped cross-correlation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("K,s,p,d", [(3, 1, 1, 1), (3, 2, 1, 1), (3, 1, 2, 2), (5, 1, 2, 1),
                                     (1, 1, 0, 1), (3, 2, 0, 2)])
def test_zero_offsets_equal_depthwise_conv2d(K, s, p, d):
    rng = np.random.default_rng(10 + K * 7 + s * 3 + p + d)
    N, Hh, Ww, G, Cg = 2, 9, 8, 3, 4
    P = K * K
    Ho, Wo = H.out_dim(Hh, K, s, p, d), H.out_dim(Ww, K, s, p, d)
    x = rng.standard_normal((N, Hh, Ww, G * Cg))
    wk = rng.standard_normal((G, P))                      # one weight per group and point
    off = np.zeros((N, Ho, Wo, G * 2 * P))
    m = np.broadcast_to(wk.reshape(1, 1, 1, G * P), (N, Ho, Wo, G * P)).copy()
    got = run64(x, off, m, K=K, stride=s, pad=p, dil=d)
    weight = torch.from_numpy(np.repeat(wk.reshape(G, 1, K, K), Cg, axis=0))   # [C,1,K,K]
    ref_nchw = torch.nn.functional.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2), weight,
                                          stride=s, padding=p, dilation=d, groups=G * Cg)
    np.testing.assert_allclose(got, ref_nchw.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)
    got32 = run32(x.astype(np.float32), off, m.astype(np.float32), K=K, stride=s, pad=p, dil=d)
    np.testing.assert_allclose(got32, ref_nchw.permute(0, 2, 3, 1).numpy(), rtol=0, atol=2e-5)


def test_zero_offsets_per_pixel_weights_shifted_window_sum():
    rng = np.random.default_rng(3)
    N, Hh, Ww, G, Cg, K, s, p, d = 1, 7, 9, 2, 3, 3, 1, 1, 1
    P = K * K
    x = rng.standard_normal((N, Hh, Ww, G * Cg))
    m = rng.standard_normal((N, Hh, Ww, G * P))
    off = np.zeros((N, Hh, Ww, G * 2 * P))
    got = run64(x, off, m, K=K, stride=s, pad=p, dil=d)
    xp = np.pad(x, ((0, 0), (1, 1), (1, 1), (0, 0)))
    want = np.zeros_like(x)
    for g in range(G):
        for k in range(P):
            i, j = divmod(k, K)
            win = xp[:, i:i + Hh, j:j + Ww, g * Cg:(g + 1) * Cg]
            want[..., g * Cg:(g + 1) * Cg] += m[..., g * P + k:g * P + k + 1] * win
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# integer offsets: exact shifted gathers
# --------------------------------------------------------------------------

def test_integer_offsets_exact_gather_sum():
    """Integer data and weights keep every fp32 step exact, so the binary32
    sequence must equal the integer gather sum bit for bit."""
    rng = np.random.default_rng(4)
    N, Hh, Ww, G, Cg, K, s, p, d = 2, 8, 7, 4, 3, 3, 1, 1, 1
    P = K * K
    x = rng.integers(-64, 65, (N, Hh, Ww, G * Cg))
    off = rng.integers(-3, 4, (N, Hh, Ww, G * 2 * P))
    m = rng.integers(-8, 9, (N, Hh, Ww, G * P))
    got = run32(x, off, m, K=K, stride=s, pad=p, dil=d)
    want = np.zeros((N, Hh, Ww, G * Cg), dtype=np.int64)
    for n in range(N):
        for ho in range(Hh):
            for wo in range(Ww):
                for g in range(G):
                    for k in range(P):
                        i, j = divmod(k, K)
                        yy = ho - p + i * d + off[n, ho, wo, g * 2 * P + P + k]
                        xx = wo - p + j * d + off[n, ho, wo, g * 2 * P + k]
                        if 0 <= yy < Hh and 0 <= xx < Ww:
                            want[n, ho, wo, g * Cg:(g + 1) * Cg] += (
                                m[n, ho, wo, g * P + k] * x[n, yy, xx, g * Cg:(g + 1) * Cg])
    assert np.array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_k1_integer_offset_pure_gather_bitwise(dtype):
    rng = np.random.default_rng(5)
    N, Hh, Ww, G, Cg = 1, 6, 5, 2, 8
    xv = rng.standard_normal((N, Hh, Ww, G * Cg)).astype(np.float32)
    x = ref.from_f32(xv, dtype)
    off = rng.integers(-2, 3, (N, Hh, Ww, G * 2)).astype(np.float32)
    m = np.ones((N, Hh, Ww, G), dtype=np.float32)
    got = ref.forward_f32(x, ref.from_f32(off, dtype), ref.from_f32(m, dtype), dtype=dtype,
                          K=1, stride=1, pad=0, dil=1)
    xi = x.view(np.uint16) if dtype != "f32" else x.view(np.uint32)
    gi = got.view(xi.dtype)
    for ho in range(Hh):
        for wo in range(Ww):
            for g in range(G):
                yy, xx = ho + int(off[0, ho, wo, 2 * g + 1]), wo + int(off[0, ho, wo, 2 * g])
                want = xi[0, yy, xx, g * Cg:(g + 1) * Cg] if (0 <= yy < Hh and 0 <= xx < Ww) \
                    else np.zeros(Cg, xi.dtype)
                assert np.array_equal(gi[0, ho, wo, g * Cg:(g + 1) * Cg], want)


# --------------------------------------------------------------------------
# linear ramp, half pixel
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_linear_ramp_exact(dtype):
    """x = a*row + b*col + e is reproduced exactly at any position inside
    [0,H-1] x [0,W-1]; dyadic data keep every binary32 step exact.  a != b
    pins which offset plane moves which axis; the one-hot weights pin the
    point order."""
    rng = np.random.default_rng(6)
    Hh, Ww, G, Cg, K = 9, 11, 2, 3, 3
    P = K * K
    a = np.array([3.0, -2.0, 1.0, 5.0, 0.5, -1.0])[:G * Cg]
    b = np.array([1.0, 4.0, -3.0, 0.25, 2.0, 7.0])[:G * Cg]
    e = np.array([0.5, -1.0, 2.0, 0.0, 1.0, -3.0])[:G * Cg]
    r = np.arange(Hh)[:, None, None]
    c = np.arange(Ww)[None, :, None]
    x = (a * r + b * c + e)[None].astype(np.float64)
    for k in range(P):
        i, j = divmod(k, K)
        off = np.zeros((1, Hh, Ww, G * 2 * P))
        m = np.zeros((1, Hh, Ww, G * P))
        want = np.zeros((1, Hh, Ww, G * Cg))
        for ho in range(Hh):
            for wo in range(Ww):
                for g in range(G):
                    by, bx = ho - 1 + i, wo - 1 + j
                    ty = rng.integers(0, 4 * (Hh - 1) + 1) / 4.0   # target inside, quarter steps
                    tx = rng.integers(0, 4 * (Ww - 1) + 1) / 4.0
                    off[0, ho, wo, g * 2 * P + k] = tx - bx
                    off[0, ho, wo, g * 2 * P + P + k] = ty - by
                    m[0, ho, wo, g * P + k] = 1.0
                    sl = slice(g * Cg, (g + 1) * Cg)
                    want[0, ho, wo, sl] = a[sl] * ty + b[sl] * tx + e[sl]
        assert np.array_equal(run64(x, off, m), want)
        got = ref.forward_f32(ref.from_f32(x, dtype), ref.from_f32(off, dtype),
                              ref.from_f32(m, dtype), dtype=dtype)
        assert np.array_equal(ref.to_f32(got, dtype), ref.to_f32(ref.from_f32(want, dtype), dtype))


def test_half_pixel_means():
    rng = np.random.default_rng(7)
    Hh, Ww, Cg = 4, 5, 4
    x = rng.integers(-100, 100, (1, Hh, Ww, Cg)).astype(np.float64)
    P = 1
    for dx, dy in ((0.5, 0.0), (0.0, 0.5), (0.5, 0.5)):
        off = np.zeros((1, Hh, Ww, 2 * P))
        off[..., 0], off[..., 1] = dx, dy
        m = np.ones((1, Hh, Ww, P))
        got = run32(x, off, m, K=1, stride=1, pad=0, dil=1)
        for yy in range(Hh):
            for xx in range(Ww):
                nb = [(yy + a, xx + b) for a in (0, 1) for b in (0, 1)
                      if (a == 0 or dy) and (b == 0 or dx)]
                acc = sum(x[0, q0, q1] if (q0 < Hh and q1 < Ww) else 0.0 for q0, q1 in nb)
                assert np.array_equal(got[0, yy, xx], (acc / len(nb)).astype(np.float32))


# --------------------------------------------------------------------------
# weight linearity (no softmax), OOB, groups, offset_scale, centre removal
# --------------------------------------------------------------------------

def test_weights_scale_linearly_no_softmax():
    rng = np.random.default_rng(8)
    x, off, m = H.random_case(rng, 1, 8, 8, 2, 4, 3, 1, 1, 1)
    base = run32(x, off, m)
    assert np.array_equal(run32(x, off, 4.0 * m), 4.0 * base)
    assert np.array_equal(run32(x, off, -m), -base)
    assert np.array_equal(run32(x, off, 0.0 * m), np.zeros_like(base))
    # superposition over points (within rounding)
    P = 9
    total = np.zeros(base.shape)
    for k in range(P):
        mk = np.zeros_like(m)
        mk[..., k::P] = m[..., k::P]
        total += run64(x, off, mk)
    np.testing.assert_allclose(total, run64(x, off, m), rtol=1e-12, atol=1e-12)
    # a softmax over the points would make all-equal weights position-independent; raw weights don't
    ones = np.ones_like(m)
    assert not np.allclose(run64(x, off, 2.0 * ones), run64(x, off, ones))


def test_all_points_outside_give_exact_zero():
    rng = np.random.default_rng(9)
    N, Hh, Ww = 1, 6, 7
    x, off, m = H.random_case(rng, N, Hh, Ww, 2, 3, 3, 1, 1, 1)
    for big in (Ww + 2.0, -(Ww + 2.0), 1e30):
        o = np.full_like(off, big)
        assert np.array_equal(run32(x, o, m), np.zeros((N, Hh, Ww, 6), np.float32))
        assert np.array_equal(run64(x, o, m), np.zeros((N, Hh, Ww, 6)))
    o = np.full_like(off, np.nan)
    assert np.array_equal(run32(x, o, m), np.zeros((N, Hh, Ww, 6), np.float32))


def test_group_permutation():
    rng = np.random.default_rng(11)
    N, Hh, Ww, G, Cg, P = 1, 6, 6, 3, 2, 9
    x, off, m = H.random_case(rng, N, Hh, Ww, G, Cg, 3, 1, 1, 1)
    perm = [2, 0, 1]
    xp = np.concatenate([x[..., g * Cg:(g + 1) * Cg] for g in perm], -1)
    op = np.concatenate([off[..., g * 2 * P:(g + 1) * 2 * P] for g in perm], -1)
    mp = np.concatenate([m[..., g * P:(g + 1) * P] for g in perm], -1)
    base = run32(x, off, m)
    want = np.concatenate([base[..., g * Cg:(g + 1) * Cg] for g in perm], -1)
    assert np.array_equal(run32(xp, op, mp), want)


def test_offset_scale_is_a_multiplier():
    rng = np.random.default_rng(12)
    x, off, m = H.random_case(rng, 1, 7, 6, 2, 3, 3, 1, 1, 1)
    assert np.array_equal(run32(x, off, m, offset_scale=2.0), run32(x, 2.0 * off, m))
    assert np.array_equal(run32(x, off, m, offset_scale=0.0), run32(x, 0.0 * off, m))
    assert np.array_equal(run32(x, 4.0 * off, m, offset_scale=0.25), run32(x, off, m))


def test_remove_center_equals_zero_centre_weight():
    rng = np.random.default_rng(13)
    N, Hh, Ww, G, Cg, K = 1, 6, 7, 2, 3, 3
    P = K * K
    x, off, m = H.random_case(rng, N, Hh, Ww, G, Cg, K, 1, 1, 1)
    c = P // 2
    m0 = m.copy()
    m0[..., c::P] = 0.0
    keep = [k for k in range(P) if k != c]
    off_rc = np.concatenate([off[..., g * 2 * P + pl * P + np.array(keep)]
                             for g in range(G) for pl in (0, 1)], -1)
    m_rc = np.concatenate([m[..., g * P + np.array(keep)] for g in range(G)], -1)
    assert np.array_equal(run32(x, off_rc, m_rc, remove_center=True), run32(x, off, m0))
    np.testing.assert_allclose(run64(x, off_rc, m_rc, remove_center=True), run64(x, off, m0),
                               rtol=1e-13, atol=1e-13)


def test_packed_offset_mask_rows():
    """offset and mask read from one [.., 3*G*P] row per pixel, as the
    projection that predicts both produces them (DCNv4Block example,
    jsqmd.com/news/933833 section 2)."""
    rng = np.random.default_rng(14)
    N, Hh, Ww, G, Cg, P = 2, 5, 6, 2, 4, 9
    x, off, m = H.random_case(rng, N, Hh, Ww, G, Cg, 3, 1, 1, 1)
    packed = np.concatenate([off, m], -1).astype(np.float32)
    got = ref.forward_f32(f32(x), packed[..., :G * 2 * P], packed[..., G * 2 * P:], dtype="f32")
    assert np.array_equal(got, run32(x, off, m))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_io_rounding_is_one_final_rounding(dtype):
    """Inputs already representable in the I/O type: the I/O-typed run equals
    the binary32 run rounded once at the end."""
    rng = np.random.default_rng(15)
    x, off, m = H.random_case(rng, 2, 7, 8, 2, 8, 3, 1, 1, 1)
    xs, os_, ms = (ref.from_f32(f32(a), dtype) for a in (x, off, m))
    got = ref.forward_f32(xs, os_, ms, dtype=dtype)
    full = run32(ref.to_f32(xs, dtype), ref.to_f32(os_, dtype), ref.to_f32(ms, dtype))
    assert np.array_equal(got.view(np.uint16), ref.from_f32(full, dtype).view(np.uint16))


# --------------------------------------------------------------------------
# golden, hand-worked examples
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_golden_bilinear_k1(dtype):
    with open(os.path.join(GOLDEN, "bilinear_k1.json")) as fh:
        gd = json.load(fh)
    p = gd["params"]
    x, off, m = (np.array(gd[k], dtype=np.float64) for k in ("x", "offset", "mask"))
    want = np.array(gd["expected"], dtype=np.float64)
    kw = dict(K=p["K"], stride=p["stride"], pad=p["pad"], dil=p["dil"], offset_scale=p["offset_scale"])
    assert np.array_equal(run64(x, off, m, **kw), want)
    got = ref.forward_f32(ref.from_f32(x, dtype), ref.from_f32(off, dtype), ref.from_f32(m, dtype),
                          dtype=dtype, **kw)
    assert np.array_equal(ref.to_f32(got, dtype), want.astype(np.float32))


def test_golden_grid_k3():
    with open(os.path.join(GOLDEN, "grid_k3.json")) as fh:
        gd = json.load(fh)
    for case in gd["cases"]:
        p = case["params"]
        K = p["K"]
        P = K * K
        x = np.array(case["x_rows"], dtype=np.float64)[None, :, :, None]
        Ho, Wo = H.out_dim(p["H"], K, p["stride"], p["pad"], p["dil"]), H.out_dim(p["W"], K, p["stride"], p["pad"], p["dil"])
        off = np.zeros((1, Ho, Wo, 2 * P))
        off[..., case["offset_k"]] = case["dx"]
        off[..., P + case["offset_k"]] = case["dy"]
        m = np.zeros((1, Ho, Wo, P))
        m[..., case["mask_onehot_k"]] = 1.0
        kw = dict(K=K, stride=p["stride"], pad=p["pad"], dil=p["dil"])
        want = np.array(case["expected_rows"], dtype=np.float64)[None, :, :, None]
        assert np.array_equal(run64(x, off, m, **kw), want), case["name"]
        assert np.array_equal(run32(x, off, m, **kw), want.astype(np.float32)), case["name"]
