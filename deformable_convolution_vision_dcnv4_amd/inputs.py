"""Seeded synthetic inputs for the DCNv4 forward.

This module draws random numbers and nothing else: it holds none of the
operator's arithmetic, so both the HIP path's tests and the CPU oracle can be
fed from it.

Generator (counter-based, so any element can be produced independently):
  splitmix64's output function  mix(z) = z ^ z>>30, *0xBF58476D1CE4E5B9,
  ^ >>27, *0x94D049BB133111EB, ^ >>31  (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014), all arithmetic mod 2**64;
  key(seed, stream)  = mix(mix(seed + GOLDEN) + (stream + 1) * GOLDEN)
  word(seed, stream, i) = mix(key + (i + 1) * GOLDEN),  GOLDEN = 0x9E3779B97F4A7C15
  uniform(i) = (word >> 11) * 2**-53 in [0, 1)
  normal(i)  = sqrt(-2 ln(1 - u(2i))) * cos(2 pi u(2i+1))   (Box-Muller, float64)
Values are scaled in float64, rounded to float32 (nearest even), then to the
I/O type (nearest even).  Streams: x = 0, offset = 1, mask = 2.
Smooth offsets (a workload's offset_smooth = r > 0): the float64 offset draws,
as [N, Ho, Wo, channel], are summed over the (2r+1) x (2r+1) output pixels
around each pixel (the image wrapping around at its edges) and divided by
2r+1, so each offset is still normal with the same standard deviation while
neighbours share most of their terms; then rounded as above.
"""
import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
STREAM_X, STREAM_OFFSET, STREAM_MASK = 0, 1, 2
_CHUNK = 1 << 22


def _mix(z):
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _key(seed, stream):
    with np.errstate(over="ignore"):
        k = _mix(np.uint64(seed % (1 << 64)) + GOLDEN)
        return _mix(k + np.uint64(stream + 1) * GOLDEN)


def uniform_words(seed, stream, start, count):
    """float64 uniforms in [0,1) for counters start .. start+count-1."""
    key = _key(seed, stream)
    i = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        w = _mix(key + (i + np.uint64(1)) * GOLDEN)
    return (w >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def draw(seed, stream, count, dist):
    """float64 draws: dist = ("normal", sigma) | ("uniform", lo, hi)."""
    out = np.empty(count, dtype=np.float64)
    kind = dist[0]
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        if kind == "normal":
            u = uniform_words(seed, stream, 2 * s, 2 * n)
            u1, u2 = u[0::2], u[1::2]
            out[s:s + n] = np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * np.pi * u2) * dist[1]
        elif kind == "uniform":
            u = uniform_words(seed, stream, s, n)
            out[s:s + n] = dist[1] + (dist[2] - dist[1]) * u
        else:
            raise ValueError(f"unknown distribution {dist!r}")
    return out


def box_smooth(a, r):
    """Sum of a [N, H, W, C] float64 array over the (2r+1)^2 pixels around
    each pixel (wrapping around), divided by 2r+1."""
    rows = np.zeros_like(a)
    for dy in range(-r, r + 1):
        rows += np.roll(a, dy, axis=1)
    out = np.zeros_like(a)
    for dx in range(-r, r + 1):
        out += np.roll(rows, dx, axis=2)
    return out / (2 * r + 1)


def to_io(values_f64, dtype):
    """float64 -> float32 (RNE) -> I/O type (RNE).  bf16 comes back as uint16 bits."""
    f32 = np.asarray(values_f64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f32
    if dtype == "f16":
        return f32.astype(np.float16)
    if dtype == "bf16":
        import torch  # library rounding (nearest even) for bfloat16
        return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def make_inputs(wl, dtype, seed=None, integer_offsets=False):
    """Host arrays (x, offset, mask) for a Workload in the I/O type."""
    seed = wl.seed if seed is None else seed
    Ho, Wo = wl.out_hw()
    nx = wl.N * wl.H * wl.W * wl.C
    npix = wl.N * Ho * Wo
    x = draw(seed, STREAM_X, nx, wl.x_dist)
    off = draw(seed, STREAM_OFFSET, npix * wl.G * 2 * wl.P, wl.offset_dist)
    r = getattr(wl, "offset_smooth", 0)
    if r > 0:
        off = box_smooth(off.reshape(wl.N, Ho, Wo, wl.G * 2 * wl.P), r).reshape(-1)
    if integer_offsets:
        off = np.rint(off)
    m = draw(seed, STREAM_MASK, npix * wl.G * wl.P, wl.mask_dist)
    return (to_io(x, dtype).reshape(wl.N, wl.H, wl.W, wl.C),
            to_io(off, dtype).reshape(wl.N, Ho, Wo, wl.G * 2 * wl.P),
            to_io(m, dtype).reshape(wl.N, Ho, Wo, wl.G * wl.P))


def as_f64(a, dtype):
    """Exact float64 value of I/O-typed host data (library widening)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
