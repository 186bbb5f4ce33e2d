"""ctypes front end of the C oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  Arrays are host numpy arrays:

    x       [N, H, W, G*Cg]          channels-last input
    offset  [N, Ho, Wo, G*2*P]       per output pixel, per group (2, P): plane 0
                                     moves along W, plane 1 along H
    mask    [N, Ho, Wo, G*P]         raw dynamic weights (no softmax)
    grad_out [N, Ho, Wo, G*Cg]       (backward) gradient of the output

with P = K*K, or K*K - 1 when the centre point is removed.  The I/O type is
named by ``dtype``: "f32" (numpy float32), "f16" (numpy float16) or "bf16"
(numpy uint16 holding bfloat16 bit patterns).  ``offset`` and ``mask`` may be
views that step through a larger per-pixel row (a packed offset+mask tensor):
only their last axis must be contiguous and their pixel stride uniform.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DCNV4_ORACLE_LIB points the wrapper at another build of the same source
# (the mutation tests compile deliberately broken copies to prove the pins bite).
_LIB_PATH = os.environ.get("DCNV4_ORACLE_LIB") or os.path.join(_HERE, "libdcnv4_oracle.so")
_lib = None

DTYPES = {"f32": (0, np.float32), "f16": (1, np.float16), "bf16": (2, np.uint16)}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, f32, f64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_double)
        L.dcnv4_oracle_output_dim.argtypes = [i32] * 5
        L.dcnv4_oracle_output_dim.restype = i32
        L.dcnv4_oracle_forward_f32.argtypes = [vp, vp, vp, vp] + [i32] * 9 + [f32, i32, i64, i64, i32]
        L.dcnv4_oracle_forward_f32.restype = i32
        L.dcnv4_oracle_forward_f64.argtypes = [vp, vp, vp, vp] + [i32] * 9 + [f64, i32, i64, i64]
        L.dcnv4_oracle_forward_f64.restype = i32
        L.dcnv4_oracle_backward_f64.argtypes = [vp] * 11 + [i32] * 9 + [f64, i32, i64, i64, i32]
        L.dcnv4_oracle_backward_f64.restype = i32
        L.dcnv4_oracle_softmax_rows_f64.argtypes = [vp, vp, i64, i32, i32, i64]
        L.dcnv4_oracle_softmax_rows_f64.restype = i32
        for name in ("f16_to_f32_array", "bf16_to_f32_array", "f32_to_f16_array", "f32_to_bf16_array"):
            fn = getattr(L, "dcnv4_oracle_" + name)
            fn.argtypes = [vp, vp, i64]
            fn.restype = None
        _lib = L
    return _lib


def output_dim(n, K, stride, pad, dil):
    return lib().dcnv4_oracle_output_dim(n, K, stride, pad, dil)


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _pixel_view(a, name, itemsize):
    """Return (array, pixel stride in elements) for a 4-D per-pixel view;
    anything that is not such a view is copied to a contiguous array."""
    if a.ndim != 4:
        raise ValueError(f"{name}: need a 4-D [N, Ho, Wo, row] array")
    n, h, w, _ = a.shape
    s2 = a.strides[2]
    uniform = (a.strides[3] == itemsize and s2 > 0 and s2 % itemsize == 0 and
               a.strides[1] == s2 * w and a.strides[0] == s2 * w * h)
    if not uniform:
        a = np.ascontiguousarray(a)
        s2 = a.strides[2] if a.shape[-1] else itemsize
    return a, s2 // itemsize


def _dims(x, offset, mask, K, stride, pad, dil, remove_center, groups):
    N, H, W, C = x.shape
    P = K * K - (1 if remove_center else 0)
    G = groups if groups is not None else offset.shape[-1] // (2 * P)
    if G < 1 or C % G:
        raise ValueError("channel count is not a multiple of the group count")
    Ho, Wo = output_dim(H, K, stride, pad, dil), output_dim(W, K, stride, pad, dil)
    if offset.shape[:3] != (N, Ho, Wo) or mask.shape[:3] != (N, Ho, Wo):
        raise ValueError("offset/mask must be [N, Ho, Wo, ...]")
    if offset.shape[-1] < G * 2 * P or mask.shape[-1] < G * P:
        raise ValueError("offset/mask rows too short for the group count")
    return N, H, W, G, C // G, Ho, Wo, P


def forward_f32(x, offset, mask, *, dtype="f32", K=3, stride=1, pad=1, dil=1,
                offset_scale=1.0, remove_center=False, groups=None):
    """The binary32 operation sequence, rounded once to ``dtype``."""
    code, npdt = DTYPES[dtype]
    for name, a in (("x", x), ("offset", offset), ("mask", mask)):
        if a.dtype != npdt:
            raise TypeError(f"{name}: expected {np.dtype(npdt)} for {dtype}, got {a.dtype}")
    x = np.ascontiguousarray(x)
    N, H, W, G, Cg, Ho, Wo, P = _dims(x, offset, mask, K, stride, pad, dil, remove_center, groups)
    isz = np.dtype(npdt).itemsize
    offset, ost = _pixel_view(offset, "offset", isz)
    mask, mst = _pixel_view(mask, "mask", isz)
    out = np.zeros((N, Ho, Wo, G * Cg), dtype=npdt)
    rc = lib().dcnv4_oracle_forward_f32(_ptr(x), _ptr(offset), _ptr(mask), _ptr(out),
                                        N, H, W, G, Cg, K, stride, pad, dil,
                                        float(offset_scale), int(bool(remove_center)),
                                        ost, mst, code)
    if rc != 0:
        raise RuntimeError(f"oracle f32 failed with status {rc}")
    return out


def forward_f64(x, offset, mask, *, K=3, stride=1, pad=1, dil=1, offset_scale=1.0,
                remove_center=False, groups=None):
    """The plain definition in double precision (inputs given as float64)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if offset.dtype != np.float64 or mask.dtype != np.float64:
        raise TypeError("offset/mask must be float64")
    N, H, W, G, Cg, Ho, Wo, P = _dims(x, offset, mask, K, stride, pad, dil, remove_center, groups)
    offset, ost = _pixel_view(offset, "offset", 8)
    mask, mst = _pixel_view(mask, "mask", 8)
    out = np.zeros((N, Ho, Wo, G * Cg), dtype=np.float64)
    rc = lib().dcnv4_oracle_forward_f64(_ptr(x), _ptr(offset), _ptr(mask), _ptr(out),
                                        N, H, W, G, Cg, K, stride, pad, dil,
                                        float(offset_scale), int(bool(remove_center)), ost, mst)
    if rc != 0:
        raise RuntimeError(f"oracle f64 failed with status {rc}")
    return out


def backward_f64(x, offset, mask, grad_out, *, K=3, stride=1, pad=1, dil=1, offset_scale=1.0,
                 remove_center=False, groups=None, bounds=False, f32_positions=False):
    """Gradients of the plain definition in double precision (inputs float64).

    Returns (grad_x [N,H,W,C], grad_offset [N,Ho,Wo,G*2*P], grad_mask
    [N,Ho,Wo,G*P]).  With ``bounds``, also a dict of the absolute-value sums
    and term counts that bound a binary32 evaluation's rounding error:
    {"abs_x", "cnt_x", "abs_offset", "abs_mask"} (same shapes).  With
    ``f32_positions`` the sampling positions are the forward's binary32 ones
    (the reference for a binary32 evaluation)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    grad_out = np.ascontiguousarray(grad_out, dtype=np.float64)
    if offset.dtype != np.float64 or mask.dtype != np.float64:
        raise TypeError("offset/mask must be float64")
    N, H, W, G, Cg, Ho, Wo, P = _dims(x, offset, mask, K, stride, pad, dil, remove_center, groups)
    if grad_out.shape != (N, Ho, Wo, G * Cg):
        raise ValueError("grad_out must be [N, Ho, Wo, G*Cg]")
    offset = np.ascontiguousarray(offset[..., :G * 2 * P])
    mask = np.ascontiguousarray(mask[..., :G * P])
    gx = np.zeros(x.shape, dtype=np.float64)
    goff = np.zeros((N, Ho, Wo, G * 2 * P), dtype=np.float64)
    gm = np.zeros((N, Ho, Wo, G * P), dtype=np.float64)
    null = ctypes.c_void_p(0)
    extra = [np.zeros_like(gx), np.zeros_like(gx), np.zeros_like(goff), np.zeros_like(gm)] if bounds else None
    ptrs = [_ptr(e) for e in extra] if bounds else [null] * 4
    rc = lib().dcnv4_oracle_backward_f64(_ptr(x), _ptr(offset), _ptr(mask), _ptr(grad_out), _ptr(gx),
                                         _ptr(goff), _ptr(gm), *ptrs, N, H, W, G, Cg, K, stride, pad, dil,
                                         float(offset_scale), int(bool(remove_center)), G * 2 * P, G * P,
                                         int(bool(f32_positions)))
    if rc != 0:
        raise RuntimeError(f"oracle backward failed with status {rc}")
    if bounds:
        return gx, goff, gm, dict(zip(("abs_x", "cnt_x", "abs_offset", "abs_mask"), extra))
    return gx, goff, gm


def softmax_weights(mask, *, groups, P):
    """DCNv3's normalisation of the weights: softmax over each group's P
    points, per pixel, in double precision.  mask [N, Ho, Wo, >= G*P] float64."""
    m = np.ascontiguousarray(mask, dtype=np.float64)
    out = np.zeros_like(m)
    N, Ho, Wo, R = m.shape
    rc = lib().dcnv4_oracle_softmax_rows_f64(_ptr(m), _ptr(out), N * Ho * Wo, groups, P, R)
    if rc != 0:
        raise RuntimeError(f"oracle softmax failed with status {rc}")
    return out


def forward_softmax_f64(x, offset, mask, *, K=3, stride=1, pad=1, dil=1, offset_scale=1.0,
                        remove_center=False, groups=None):
    """The DCNv3-style aggregation: the plain definition with softmax-normalised
    weights (double precision)."""
    N, H, W, G, Cg, Ho, Wo, P = _dims(np.asarray(x), offset, mask, K, stride, pad, dil, remove_center, groups)
    w = softmax_weights(mask[..., :G * P], groups=G, P=P)
    return forward_f64(x, offset, w, K=K, stride=stride, pad=pad, dil=dil, offset_scale=offset_scale,
                       remove_center=remove_center, groups=G)


def to_f32(a, dtype):
    """Exact widening of I/O-typed values to float32 (the oracle's decoder)."""
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float32)
    if dtype == "f32":
        out[...] = a
    elif dtype == "f16":
        lib().dcnv4_oracle_f16_to_f32_array(_ptr(a.view(np.uint16)), _ptr(out), a.size)
    elif dtype == "bf16":
        lib().dcnv4_oracle_bf16_to_f32_array(_ptr(a), _ptr(out), a.size)
    else:
        raise ValueError(dtype)
    return out


def from_f32(a, dtype):
    """Round float32 values to the I/O type, nearest even (the oracle's encoder)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a.copy()
    out = np.empty(a.shape, dtype=np.uint16)
    if dtype == "f16":
        lib().dcnv4_oracle_f32_to_f16_array(_ptr(a), _ptr(out), a.size)
        return out.view(np.float16)
    if dtype == "bf16":
        lib().dcnv4_oracle_f32_to_bf16_array(_ptr(a), _ptr(out), a.size)
        return out
    raise ValueError(dtype)
