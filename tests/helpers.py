"""Test-side helpers: brute-force pins and error bounds (no operator code here
that the oracle or the HIP path shares)."""
import numpy as np

U32 = 2.0 ** -24   # unit roundoff of binary32


def gamma(n, u=U32):
    return n * u / (1.0 - n * u)


def out_dim(n, K, stride, pad, dil):
    span = n + 2 * pad - dil * (K - 1) - 1
    return span // stride + 1 if span >= 0 else 0


def point_list(K, remove_center=False):
    pts = [(i, j) for i in range(K) for j in range(K)]
    if remove_center:
        pts.remove((K // 2, K // 2))
    return pts


def bruteforce_f64(x, offset, mask, K, stride, pad, dil, scale=1.0, remove_center=False):
    """Triangle-kernel form of bilinear sampling, summed over EVERY pixel.

    Bilinear interpolation with zero padding equals
      sum_q max(0, 1-|py-qy|) * max(0, 1-|px-qx|) * f(q)
    over all pixels q of the image; this evaluates that sum directly (tiny
    inputs only) instead of locating the four corners.
    """
    x = np.asarray(x, dtype=np.float64)
    N, H, W, C = x.shape
    pts = point_list(K, remove_center)
    P = len(pts)
    G = offset.shape[-1] // (2 * P)
    Cg = C // G
    Ho, Wo = out_dim(H, K, stride, pad, dil), out_dim(W, K, stride, pad, dil)
    qy = np.arange(H, dtype=np.float64)[:, None]
    qx = np.arange(W, dtype=np.float64)[None, :]
    out = np.zeros((N, Ho, Wo, C), dtype=np.float64)
    for n in range(N):
        for ho in range(Ho):
            for wo in range(Wo):
                for g in range(G):
                    acc = np.zeros(Cg)
                    for k, (i, j) in enumerate(pts):
                        dx = offset[n, ho, wo, g * 2 * P + k]
                        dy = offset[n, ho, wo, g * 2 * P + P + k]
                        m = mask[n, ho, wo, g * P + k]
                        py = ho * stride - pad + i * dil + scale * dy
                        px = wo * stride - pad + j * dil + scale * dx
                        wgt = np.maximum(0.0, 1.0 - np.abs(py - qy)) * np.maximum(0.0, 1.0 - np.abs(px - qx))
                        acc += m * np.tensordot(wgt, x[n, :, :, g * Cg:(g + 1) * Cg], axes=([0, 1], [0, 1]))
                    out[n, ho, wo, g * Cg:(g + 1) * Cg] = acc
    return out


def f32_bound(x64, offset64, mask64, K, stride, pad, dil, scale=1.0, remove_center=False):
    """Per-output bound on |binary32 sequence - exact value|.

    Position: one rounding in the fma, |dp| <= u*(|p| + 1) per axis with the
    fraction/complement roundings folded in; the bilinear sample moves by at
    most 2*vmax per unit of position.  Weights carry <= 4 roundings, the
    accumulation 4P fmas: gamma(4P + 4) * sum |m| * vmax.  Doubled for slack.
    """
    N, H, W, C = x64.shape
    P = K * K - (1 if remove_center else 0)
    G = offset64.shape[-1] // (2 * P)
    Cg = C // G
    vmax = float(np.max(np.abs(x64))) if x64.size else 0.0
    pmax = max(H, W) * stride + pad + dil * K + abs(scale) * float(np.max(np.abs(offset64), initial=0.0))
    per_pt = 2.0 * vmax * 2.0 * U32 * (pmax + 2.0) + gamma(4 * P + 4) * vmax
    msum = np.abs(mask64.reshape(mask64.shape[:3] + (-1,))[..., :G * P]).reshape(
        mask64.shape[:3] + (G, P)).sum(-1)                       # [N,Ho,Wo,G]
    bound = 2.0 * per_pt * msum
    return np.repeat(bound, Cg, axis=-1)


def random_case(rng, N, H, W, G, Cg, K, stride, pad, dil, off_sigma=1.5, remove_center=False):
    """float64 inputs that are exactly representable in binary32."""
    P = K * K - (1 if remove_center else 0)
    Ho, Wo = out_dim(H, K, stride, pad, dil), out_dim(W, K, stride, pad, dil)
    x = rng.standard_normal((N, H, W, G * Cg)).astype(np.float32).astype(np.float64)
    off = (rng.standard_normal((N, Ho, Wo, G * 2 * P)) * off_sigma).astype(np.float32).astype(np.float64)
    m = rng.standard_normal((N, Ho, Wo, G * P)).astype(np.float32).astype(np.float64)
    return x, off, m


def edge_offsets(rng, N, H, W, G, K, stride, pad, dil, remove_center=False):
    """Offsets that land sampling points in the border bands: just inside -1,
    exactly -1, (-1,0), (n-1,n), exactly n-1 and exactly n, per axis."""
    pts = point_list(K, remove_center)
    P = len(pts)
    Ho, Wo = out_dim(H, K, stride, pad, dil), out_dim(W, K, stride, pad, dil)
    off = np.zeros((N, Ho, Wo, G * 2 * P), dtype=np.float64)

    def target(n_ext):
        choices = np.array([-1.0, -0.75, -0.5, -0.25, -2.0 ** -20, 0.0,
                            n_ext - 1.0, n_ext - 0.5, n_ext - 2.0 ** -20, float(n_ext), n_ext + 0.25])
        return choices[rng.integers(0, len(choices))]

    for n in range(N):
        for ho in range(Ho):
            for wo in range(Wo):
                for g in range(G):
                    for k, (i, j) in enumerate(pts):
                        by = ho * stride - pad + i * dil
                        bx = wo * stride - pad + j * dil
                        ty = target(H) if rng.random() < 0.6 else by + rng.uniform(-1.5, 1.5)
                        tx = target(W) if rng.random() < 0.6 else bx + rng.uniform(-1.5, 1.5)
                        off[n, ho, wo, g * 2 * P + k] = np.float32(tx - bx)
                        off[n, ho, wo, g * 2 * P + P + k] = np.float32(ty - by)
    return off
