"""The module's C ABI on the CPU: workspace layout and validation before any
HIP call (fake device addresses, never dereferenced)."""
import ctypes

import pytest
import torch

from deformable_convolution_vision_dcnv4_amd import binding

OK, ERR_NULL, ERR_SHAPE, ERR_PARAM, ERR_DTYPE, ERR_ALIAS, ERR_TOO_LARGE, ERR_HIP, ERR_ALIGN = range(9)
X, OUT, WS = 0x10000000, 0x20000000, 0x40000000
WBASE = 0x30000000


def cfg(raw=None, **kw):
    a = dict(Cin=32, G=4, Cg=16, norm=binding.NORM_GROUP, norm_groups=32)
    a.update(kw)
    c = binding.module_config(**a)
    for k, v in (raw or {}).items():
        setattr(c, k, v)
    return c


def weights(**kw):
    w = binding.ModuleWeights()
    for i, (name, _) in enumerate(w._fields_):
        setattr(w, name, WBASE + i * 0x100000)
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def call(c=None, w=None, N=2, H=8, W=8, x=X, out=OUT, ws=WS, ws_bytes=1 << 26, dtype=1):
    c = c or cfg()
    w = w or weights()
    return binding.lib().dcnv4_module_forward(x, ctypes.byref(w), out, N, H, W, ctypes.byref(c), ws, ws_bytes,
                                              dtype, None)


def test_layout_regions_are_aligned_and_sized():
    c = cfg(center_scale=True, out_proj=True, Cout=24)
    lay = binding.module_layout(2, 9, 11, c, torch.float16)
    M, C = 2 * 9 * 11, 64
    P, G = 9, 4
    R = 3 * G * P + G
    assert lay["rows_stride"] == (R + 7) // 8 * 8
    regions = [lay[k] for k in ("xp", "xn", "d", "rows", "y", "gated", "stats")]
    assert all(r >= 0 and r % 256 == 0 for r in regions)
    assert regions == sorted(regions)
    assert lay["xn"] - lay["xp"] >= M * C * 2 and lay["y"] - lay["rows"] >= M * lay["rows_stride"] * 2
    assert lay["total"] >= lay["stats"] + 2 * 4 * 32
    # without normalisation, gate or projection the optional regions are absent
    lay2 = binding.module_layout(2, 9, 11, cfg(norm=binding.NORM_NONE), torch.float32)
    assert lay2["xn"] == lay2["y"] == lay2["gated"] == lay2["stats"] == -1
    # remove_center: P = 8
    lay3 = binding.module_layout(1, 4, 4, cfg(remove_center=True), torch.float32)
    assert lay3["rows_stride"] == (3 * 4 * 8 + 7) // 8 * 8


@pytest.mark.parametrize("kw,status", [
    (dict(c=cfg(norm_groups=5)), ERR_PARAM), (dict(c=cfg(norm=3)), ERR_PARAM),
    (dict(c=cfg(eps=0.0)), ERR_PARAM), (dict(c=cfg(Cin=30)), ERR_SHAPE), (dict(c=cfg(Cin=30), dtype=0), OK),
    (dict(c=cfg(out_proj=False, Cout=7)), ERR_SHAPE), (dict(c=cfg(out_proj=True, Cout=0)), ERR_SHAPE),
    (dict(c=cfg(G=0)), ERR_SHAPE), (dict(c=cfg(Cin=8192)), ERR_TOO_LARGE), (dict(dtype=9), ERR_DTYPE),
    (dict(c=cfg(offset_scale=float("inf"))), ERR_PARAM), (dict(c=cfg(raw=dict(remove_center=2))), ERR_PARAM),
    (dict(x=0), ERR_NULL), (dict(out=0), ERR_NULL), (dict(ws=0), ERR_NULL), (dict(w=weights(w_pred=0)), ERR_NULL),
    (dict(w=weights(gamma=0)), ERR_NULL), (dict(c=cfg(norm=binding.NORM_NONE), w=weights(gamma=0, beta=0)), OK),
    (dict(c=cfg(out_proj=True, Cout=16), w=weights(w_out=0)), ERR_NULL),
    (dict(ws_bytes=1024), ERR_TOO_LARGE), (dict(ws=WS + 64), ERR_ALIGN), (dict(x=X + 2), ERR_ALIGN),
    (dict(out=X + 256), ERR_ALIAS), (dict(ws=X), ERR_ALIAS), (dict(w=weights(b_in=WS + 4096)), ERR_ALIAS),
    (dict(N=0, x=0, out=0, ws=0), OK),
])
def test_module_validation_before_any_hip_call(kw, status):
    st = call(**kw)
    if status == OK and kw.get("N", 2) != 0:
        # valid arguments reach the device check, which fails without a GPU
        assert st in (OK, ERR_HIP)
    else:
        assert st == status, binding.last_error()
