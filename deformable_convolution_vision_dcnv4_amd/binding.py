"""Python binding of libdcnv4.so (argument marshalling only).

Every step of the operator runs in the HIP kernels behind the C ABI of
include/dcnv4.h; this module checks tensors, allocates the output with torch,
passes device pointers and torch's current HIP stream, and turns a nonzero
status into an exception.  There is no fallback: without the built library,
or without a gfx950 GPU, calls fail loudly.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdcnv4.so")
_lib = None

F32, F16, BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

# Every symbol include/dcnv4.h declares.
EXPORTS = ("dcnv4_forward", "dcnv4_forward_ex", "dcnv4_forward_softmax", "dcnv4_backward", "dcnv4_output_dim",
           "dcnv4_status_string", "dcnv4_last_error", "dcnv4_version", "dcnv4_query_plan",
           "dcnv4_query_backward_plan", "dcnv4_kernel_name", "dcnv4_module_workspace_layout",
           "dcnv4_module_forward", "dcnv4_module_forward_noalloc")

MODULE_SCRATCH_BYTES = 64 << 20   # DCNV4_MODULE_SCRATCH_BYTES

NORM_NONE, NORM_GROUP, NORM_LAYER = 0, 1, 2


class ModuleConfig(ctypes.Structure):
    _fields_ = [("Cin", ctypes.c_int), ("G", ctypes.c_int), ("Cg", ctypes.c_int), ("Cout", ctypes.c_int),
                ("norm", ctypes.c_int), ("norm_groups", ctypes.c_int), ("eps", ctypes.c_float),
                ("remove_center", ctypes.c_int), ("center_scale", ctypes.c_int), ("out_proj", ctypes.c_int),
                ("offset_scale", ctypes.c_float)]


class ModuleWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in ("w_in", "b_in", "gamma", "beta", "w_dw", "b_dw", "w_pred",
                                                     "b_pred", "w_out", "b_out")]


class ModuleLayout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in ("xp", "xn", "d", "rows", "y", "gated", "stats", "rows_stride",
                                                    "total")]


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("vec", ctypes.c_int), ("lanes_per_unit", ctypes.c_int),
                ("block", ctypes.c_int), ("grid", ctypes.c_int64), ("groups_per_block", ctypes.c_int),
                ("tile_h", ctypes.c_int), ("tile_w", ctypes.c_int), ("margin_y", ctypes.c_int),
                ("margin_x", ctypes.c_int), ("window_h", ctypes.c_int), ("window_w", ctypes.c_int),
                ("full_window", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("coalesced_offsets", ctypes.c_int), ("shared_coefficients", ctypes.c_int)]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["kernel"] = lib().dcnv4_kernel_name(self.kernel).decode()
        return d


class BackwardPlan(ctypes.Structure):
    _fields_ = [("x_path", ctypes.c_int), ("x_channels", ctypes.c_int), ("x_tile", ctypes.c_int),
                ("x_margin", ctypes.c_int), ("x_lds_bytes", ctypes.c_int), ("om_path", ctypes.c_int),
                ("om_tile_h", ctypes.c_int), ("om_tile_w", ctypes.c_int), ("om_lds_bytes", ctypes.c_int)]

    X_PATHS = ("none", "lds_whole", "lds_tiles", "atomics")
    OM_PATHS = ("none", "lds_window", "global")

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["x_path"] = self.X_PATHS[self.x_path]
        d["om_path"] = self.OM_PATHS[self.om_path]
        return d


class DCNv4Error(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"dcnv4: {status_string(status)} (status {status}): {detail}")
        self.status = status


def lib():
    """Load libdcnv4.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m deformable_convolution_vision_dcnv4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.dcnv4_forward.argtypes = [vp, vp, vp, vp] + [i32] * 9 + [f32, i32, vp]
        L.dcnv4_forward.restype = i32
        L.dcnv4_forward_ex.argtypes = [vp, vp, vp, vp] + [i32] * 9 + [f32, i32, i64, i64, i32, vp]
        L.dcnv4_forward_ex.restype = i32
        L.dcnv4_forward_softmax.argtypes = [vp, vp, vp, vp] + [i32] * 9 + [f32, i32, i64, i64, i32, vp]
        L.dcnv4_forward_softmax.restype = i32
        L.dcnv4_backward.argtypes = [vp] * 7 + [i32] * 9 + [f32, i32, i64, i64, i32, vp]
        L.dcnv4_backward.restype = i32
        L.dcnv4_output_dim.argtypes = [i32] * 5
        L.dcnv4_output_dim.restype = i32
        L.dcnv4_status_string.argtypes = [i32]
        L.dcnv4_status_string.restype = ctypes.c_char_p
        L.dcnv4_last_error.argtypes = []
        L.dcnv4_last_error.restype = ctypes.c_char_p
        L.dcnv4_version.argtypes = []
        L.dcnv4_version.restype = ctypes.c_char_p
        L.dcnv4_query_plan.argtypes = [vp, vp, vp, vp] + [i32] * 9 + [f32, i32, i64, i64, i32,
                                                                       ctypes.POINTER(Plan)]
        L.dcnv4_query_plan.restype = i32
        L.dcnv4_query_backward_plan.argtypes = [vp] * 4 + [i32] * 11 + [f32, i32, i64, i64, i32,
                                                                          ctypes.POINTER(BackwardPlan)]
        L.dcnv4_query_backward_plan.restype = i32
        L.dcnv4_module_workspace_layout.argtypes = [i32, i32, i32, ctypes.POINTER(ModuleConfig), i32,
                                                     ctypes.POINTER(ModuleLayout)]
        L.dcnv4_module_workspace_layout.restype = i32
        L.dcnv4_module_forward.argtypes = [vp, ctypes.POINTER(ModuleWeights), vp, i32, i32, i32,
                                           ctypes.POINTER(ModuleConfig), vp, ctypes.c_size_t, i32, vp]
        L.dcnv4_module_forward.restype = i32
        L.dcnv4_module_forward_noalloc.argtypes = [vp, ctypes.POINTER(ModuleWeights), vp, i32, i32, i32,
                                                   ctypes.POINTER(ModuleConfig), i32, vp]
        L.dcnv4_module_forward_noalloc.restype = i32
        L.dcnv4_kernel_name.argtypes = [i32]
        L.dcnv4_kernel_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status):
    return lib().dcnv4_status_string(int(status)).decode()


def last_error():
    return lib().dcnv4_last_error().decode()


def version():
    return lib().dcnv4_version().decode()


def output_dim(n, K, stride, pad, dilation):
    return lib().dcnv4_output_dim(n, K, stride, pad, dilation)


def _check(status):
    if status != 0:
        raise DCNv4Error(status, last_error())


def _row_view(t, name):
    """(pointer, row stride in elements) of a [N, Ho, Wo, row] tensor whose last
    axis is contiguous and whose pixels are evenly spaced."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [N, Ho, Wo, ...], got shape {tuple(t.shape)}")
    n, h, w, r = t.shape
    st = t.stride()
    if r > 1 and st[3] != 1:
        raise ValueError(f"{name}: last axis must be contiguous")
    if not (st[1] == st[2] * w and st[0] == st[1] * h) and t.numel() > 0:
        raise ValueError(f"{name}: pixels must be evenly spaced (got strides {st})")
    return t.data_ptr(), st[2]


def _prepare(x, offset, mask, kernel_size, remove_center, group, out):
    if x.dim() != 4:
        raise ValueError(f"x must be [N, H, W, C] channels-last, got shape {tuple(x.shape)}")
    if x.dtype not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {x.dtype}; use float32, float16 or bfloat16")
    for name, t in (("offset", offset), ("mask", mask)):
        if t.dtype != x.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from x dtype {x.dtype}")
        if t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")
    if x.device.type != "cuda":
        raise ValueError("tensors must be on a GPU (cuda/HIP device)")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous channels-last [N, H, W, C]")
    N, H, W, C = x.shape
    K = int(kernel_size)
    P = K * K - (1 if remove_center else 0)
    G = int(group) if group is not None else offset.shape[-1] // (2 * P)
    if G < 1 or C % G:
        raise ValueError(f"channels C={C} not divisible into G={G} groups")
    if offset.shape[-1] < G * 2 * P or mask.shape[-1] < G * P:
        raise ValueError(f"offset rows need G*2*P={G * 2 * P} and mask rows G*P={G * P} elements")
    return N, H, W, C, G, K, P


def forward(x, offset, mask, *, kernel_size=3, stride=1, pad=1, dilation=1, offset_scale=1.0,
            remove_center=False, group=None, out=None, stream=None, softmax=False):
    """DCNv4 spatial-aggregation forward on the GPU.

    x       [N, H, W, G*Cg]        channels-last, contiguous
    offset  [N, Ho, Wo, >= G*2*P]  per group K*K (or K*K-1) x-offsets then y-offsets
    mask    [N, Ho, Wo, >= G*P]    raw dynamic weights (no softmax)
    Returns out [N, Ho, Wo, G*Cg] in x's dtype (written into ``out`` if given).
    ``offset``/``mask`` may be views into one packed [N, Ho, Wo, 3*G*P] tensor.
    ``softmax``: the DCNv3-style aggregation (weights softmax-normalised over
    each group's points first).
    G defaults to offset.shape[-1] // (2*P).  The kernel runs on ``stream``
    (default: torch's current stream on x's device).
    """
    N, H, W, C, G, K, P = _prepare(x, offset, mask, kernel_size, remove_center, group, out)
    Ho, Wo = output_dim(H, K, stride, pad, dilation), output_dim(W, K, stride, pad, dilation)
    if Ho < 1 or Wo < 1:
        raise ValueError(f"no output for H={H} W={W} K={K} stride={stride} pad={pad} dilation={dilation}")
    if tuple(offset.shape[:3]) != (N, Ho, Wo) or tuple(mask.shape[:3]) != (N, Ho, Wo):
        raise ValueError(f"offset/mask must be [N, Ho, Wo, ...] = [{N}, {Ho}, {Wo}, ...]")
    if out is None:
        out = torch.empty((N, Ho, Wo, C), dtype=x.dtype, device=x.device)
    elif (tuple(out.shape) != (N, Ho, Wo, C) or out.dtype != x.dtype or not out.is_contiguous()
          or out.device != x.device):
        raise ValueError("out must be a contiguous [N, Ho, Wo, C] tensor of x's dtype and device")
    optr, orow = _row_view(offset, "offset")
    mptr, mrow = _row_view(mask, "mask")
    if stream is None:
        with torch.cuda.device(x.device):
            stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(x.device):
        if softmax:
            _check(lib().dcnv4_forward_softmax(x.data_ptr(), optr, mptr, out.data_ptr(), N, H, W, G, C // G,
                                               K, stride, pad, dilation, float(offset_scale),
                                               1 if remove_center else 0, orow, mrow,
                                               _DTYPE_CODE[x.dtype], sptr))
        elif not remove_center and orow == G * 2 * P and mrow == G * P:
            _check(lib().dcnv4_forward(x.data_ptr(), optr, mptr, out.data_ptr(), N, H, W, G, C // G,
                                       K, stride, pad, dilation, float(offset_scale),
                                       _DTYPE_CODE[x.dtype], sptr))
        else:
            _check(lib().dcnv4_forward_ex(x.data_ptr(), optr, mptr, out.data_ptr(), N, H, W, G,
                                          C // G, K, stride, pad, dilation, float(offset_scale),
                                          1 if remove_center else 0, orow, mrow,
                                          _DTYPE_CODE[x.dtype], sptr))
    return out


def backward(x, offset, mask, grad_out, *, kernel_size=3, stride=1, pad=1, dilation=1, offset_scale=1.0,
             remove_center=False, group=None, need=("x", "offset", "mask"), stream=None):
    """Gradients of `forward` given grad_out = dL/dout [N, Ho, Wo, G*Cg] (x's dtype).

    Returns (grad_x, grad_offset, grad_mask), float32, shaped like x, offset
    and mask (None for those not in ``need``).  A gradient of an offset/mask
    view into a packed tensor is returned with the view's row stride (a view
    into a new packed float32 tensor)."""
    N, H, W, C, G, K, P = _prepare(x, offset, mask, kernel_size, remove_center, group, None)
    Ho, Wo = output_dim(H, K, stride, pad, dilation), output_dim(W, K, stride, pad, dilation)
    if tuple(grad_out.shape) != (N, Ho, Wo, C) or grad_out.dtype != x.dtype or not grad_out.is_contiguous():
        raise ValueError(f"grad_out must be a contiguous [{N}, {Ho}, {Wo}, {C}] tensor of x's dtype")
    optr, orow = _row_view(offset, "offset")
    mptr, mrow = _row_view(mask, "mask")
    dev = x.device
    gx = torch.empty(x.shape, dtype=torch.float32, device=dev) if "x" in need else None
    # gradients of the rows, with the inputs' row strides
    if orow == mrow and mptr - optr == G * 2 * P * x.element_size() and ("offset" in need or "mask" in need):
        rows = torch.zeros((N, Ho, Wo, orow), dtype=torch.float32, device=dev)
        goff_full, gm_full = rows, rows[..., G * 2 * P:]
    else:
        goff_full = torch.zeros((N, Ho, Wo, orow), dtype=torch.float32, device=dev) if "offset" in need else None
        gm_full = torch.zeros((N, Ho, Wo, mrow), dtype=torch.float32, device=dev) if "mask" in need else None
    if "offset" not in need:
        goff_full = None
    if "mask" not in need:
        gm_full = None
    if stream is None:
        with torch.cuda.device(dev):
            stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)

    def ptr(t):
        return t.data_ptr() if t is not None else None

    with torch.cuda.device(dev):
        _check(lib().dcnv4_backward(x.data_ptr(), optr, mptr, grad_out.data_ptr(), ptr(gx), ptr(goff_full),
                                    ptr(gm_full), N, H, W, G, C // G, K, stride, pad, dilation,
                                    float(offset_scale), 1 if remove_center else 0, orow, mrow,
                                    _DTYPE_CODE[x.dtype], sptr))
    goff = goff_full[..., :offset.shape[-1]] if goff_full is not None else None
    gm = gm_full[..., :mask.shape[-1]] if gm_full is not None else None
    return gx, goff, gm


def forward_raw(x_ptr, offset_ptr, mask_ptr, out_ptr, N, H, W, G, Cg, K, stride, pad, dilation,
                offset_scale, dtype_code, stream_ptr):
    """The plain dcnv4_forward entry point with raw device pointers."""
    _check(lib().dcnv4_forward(x_ptr, offset_ptr, mask_ptr, out_ptr, N, H, W, G, Cg, K, stride, pad,
                               dilation, float(offset_scale), dtype_code, stream_ptr))


def query_plan(x, offset, mask, out, *, kernel_size=3, stride=1, pad=1, dilation=1,
               offset_scale=1.0, remove_center=False, group=None):
    """The launch plan the library picks for these tensors (host only)."""
    N, H, W, C, G, K, P = _prepare(x, offset, mask, kernel_size, remove_center, group, out)
    optr, orow = _row_view(offset, "offset")
    mptr, mrow = _row_view(mask, "mask")
    pl = Plan()
    _check(lib().dcnv4_query_plan(x.data_ptr(), optr, mptr, out.data_ptr(), N, H, W, G, C // G, K,
                                  stride, pad, dilation, float(offset_scale),
                                  1 if remove_center else 0, orow, mrow, _DTYPE_CODE[x.dtype],
                                  ctypes.byref(pl)))
    return pl.as_dict()


def query_backward_plan(x, offset, mask, grad_out, *, kernel_size=3, stride=1, pad=1, dilation=1,
                        offset_scale=1.0, remove_center=False, group=None, need=("x", "offset", "mask")):
    """The kernels the backward picks for these tensors (host only)."""
    N, H, W, C, G, K, P = _prepare(x, offset, mask, kernel_size, remove_center, group, None)
    optr, orow = _row_view(offset, "offset")
    mptr, mrow = _row_view(mask, "mask")
    pl = BackwardPlan()
    _check(lib().dcnv4_query_backward_plan(x.data_ptr(), optr, mptr, grad_out.data_ptr(), int("x" in need),
                                           int("offset" in need or "mask" in need), N, H, W, G, C // G, K,
                                           stride, pad, dilation, float(offset_scale),
                                           1 if remove_center else 0, orow, mrow, _DTYPE_CODE[x.dtype],
                                           ctypes.byref(pl)))
    return pl.as_dict()


def module_config(*, Cin, G, Cg, Cout=None, norm=NORM_GROUP, norm_groups=32, eps=1e-5, remove_center=False,
                  center_scale=False, out_proj=False, offset_scale=1.0):
    """The module's options as the C struct (Cout defaults to G*Cg)."""
    return ModuleConfig(int(Cin), int(G), int(Cg), int(Cout if Cout is not None else G * Cg), int(norm),
                        int(norm_groups), float(eps), int(bool(remove_center)), int(bool(center_scale)),
                        int(bool(out_proj)), float(offset_scale))


def module_layout(N, H, W, cfg, dtype):
    """Workspace layout (dict of byte offsets, -1 for unused regions)."""
    lay = ModuleLayout()
    _check(lib().dcnv4_module_workspace_layout(int(N), int(H), int(W), ctypes.byref(cfg), _DTYPE_CODE[dtype],
                                               ctypes.byref(lay)))
    return {name: getattr(lay, name) for name, _ in lay._fields_}


def module_forward(x, weights, cfg, *, out=None, workspace=None, stream=None):
    """DCNv4 module forward (include/dcnv4_module.h) on x [N, H, W, Cin].

    weights: dict of tensors on x's device -- w_in [C, Cin], w_pred [R, C],
    w_out [Cout, C] in x's dtype; b_in, gamma, beta, w_dw [C, 3, 3], b_dw,
    b_pred, b_out in float32 (gamma/beta, w_out/b_out only when used).
    Returns (out [N, H, W, Cout], workspace, layout); the workspace (a uint8
    tensor, allocated here unless given) holds the intermediates at the
    layout's byte offsets."""
    if x.dim() != 4 or not x.is_contiguous() or x.dtype not in _DTYPE_CODE:
        raise ValueError("x must be a contiguous [N, H, W, Cin] tensor of float32, float16 or bfloat16")
    N, H, W, Cin = x.shape
    if Cin != cfg.Cin:
        raise ValueError(f"x has {Cin} channels, the config {cfg.Cin}")
    lay = module_layout(N, H, W, cfg, x.dtype)
    if out is None:
        out = torch.empty((N, H, W, cfg.Cout), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(lay["total"], 256), dtype=torch.uint8, device=x.device)
    wts = ModuleWeights()
    for name, _ in wts._fields_:
        t = weights.get(name)
        if t is not None:
            if t.device != x.device or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous tensor on {x.device}")
            setattr(wts, name, t.data_ptr())
    if stream is None:
        with torch.cuda.device(x.device):
            stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(x.device):
        _check(lib().dcnv4_module_forward(x.data_ptr(), ctypes.byref(wts), out.data_ptr(), N, H, W,
                                          ctypes.byref(cfg), workspace.data_ptr(), workspace.numel(),
                                          _DTYPE_CODE[x.dtype], sptr))
    return out, workspace, lay
