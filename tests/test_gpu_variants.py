"""GPU parity for the operator's variants and for each launch path.

Variants named by the pages: dropping the centre sampling point
("掌握DCNv4技术：3倍速度提升与80%加速效果的实战指南", pwwt.cn/news/2159231,
section "进阶优化建议"), and offsets and weights read in place from one packed
per-pixel row, as the single projection of the DCNv4Block example predicts
them ("不只是卷积的平替：我把DCNv4塞进Stable Diffusion的U-Net里",
jsqmd.com/news/933833, section 2).  Every case is compared bit for bit with
the oracle's binary32 sequence, for each kernel family the planner can pick:
whole-image LDS windows, row bands with the global-memory fallback for
points that leave the band, and the direct kernel.
"""
import numpy as np
import pytest
import torch

from deformable_convolution_vision_dcnv4_amd import binding
from deformable_convolution_vision_dcnv4_amd import inputs as gen
from deformable_convolution_vision_dcnv4_amd.workloads import Workload
from oracle import ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    binding.lib()
    yield


def okw(wl):
    return dict(K=wl.K, stride=wl.stride, pad=wl.pad, dil=wl.dil, offset_scale=wl.offset_scale,
                remove_center=wl.remove_center)


def gkw(wl):
    return dict(kernel_size=wl.K, stride=wl.stride, pad=wl.pad, dilation=wl.dil,
                offset_scale=wl.offset_scale, remove_center=wl.remove_center)


# (name, N, H, W, G, Cg, offset std, dtypes, expected kernel family, full
# window, DCNV4_TUNE).  Units of three or more 16-byte vectors (fp32 Cg=16,
# 16-bit Cg=24/32/40) take one lane per vector; window_gb holds several groups
# per workgroup.  These batches are too small to fill the GPU, where the
# planner picks the direct kernel: "kernel=window" keeps the window family's
# own choices (whole image, bands, groups per workgroup) for them.
PATHS = [
    ("window_full", 2, 12, 13, 4, 16, 2.0, ("f32", "f16", "bf16"), "window", 1, "kernel=window"),
    ("window_gb", 2, 6, 7, 4, 16, 2.0, ("f32", "bf16"), "window", 1, "kernel=window"),
    ("window_full40", 2, 20, 22, 2, 40, 2.0, ("f16", "bf16"), "window", 1, "kernel=window"),
    ("window_bands24", 2, 60, 60, 1, 24, 6.0, ("f16",), "window", 0, "kernel=window"),
    ("window_bands", 2, 60, 60, 1, 16, 8.0, ("f32",), "window", 0, "kernel=window"),
    ("window_bands16", 2, 60, 60, 2, 32, 6.0, ("f16", "bf16"), "window", 0, "kernel=window"),
    ("window_fill_bands", 16, 28, 24, 4, 16, 2.0, ("f16",), "window", 0, ""),
    ("window_coal_bands_fallback", 2, 60, 60, 1, 16, 8.0, ("f16", "bf16"), "window", 0, "kernel=window,full=0"),
    ("direct", 2, 12, 13, 4, 6, 2.0, ("f32", "f16", "bf16"), "direct", 0, ""),
    ("direct_small_batch", 2, 12, 13, 4, 16, 2.0, ("f32", "f16"), "direct", 0, ""),
]
CASES = [(p, dt, rc) for p in PATHS for dt in p[7] for rc in (False, True)]


def _ids(c):
    p, dt, rc = c
    return f"{p[0]}-{dt}-{'rc' if rc else 'all'}"


def _plan(wl, dtype, x, off, m):
    xs, os_, ms = gu.dev(x, dtype), gu.dev(off, dtype), gu.dev(m, dtype)
    return binding.query_plan(xs, os_, ms, torch.empty_like(xs), **gkw(wl))


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_paths_and_remove_center_bit_exact(case, monkeypatch):
    (name, N, H, W, G, Cg, std, _, family, full, tune), dtype, rc = case
    if tune:
        monkeypatch.setenv("DCNV4_TUNE", tune)
    else:
        monkeypatch.delenv("DCNV4_TUNE", raising=False)
    wl = Workload(name, N, H, W, G, Cg, (dtype,), offset_dist=("normal", std), mask_dist=("normal", 0.7),
                  remove_center=rc, seed=21)
    x, off, m = gen.make_inputs(wl, dtype)
    plan = _plan(wl, dtype, x, off, m)
    gu.announce(f"{name} {wl.describe(dtype)} remove_center={rc} plan {plan}")
    assert plan["kernel"] == family and plan["full_window"] == full
    want = ref.forward_f32(x, off, m, dtype=dtype, **okw(wl))
    out = binding.forward(gu.dev(x, dtype), gu.dev(off, dtype), gu.dev(m, dtype), **gkw(wl))
    torch.cuda.synchronize()
    got = gu.host(out, dtype)
    gu.compare(got, want, dtype, label=name)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("tune", ["", "kernel=window"], ids=["auto", "window"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rc", [False, True])
@pytest.mark.parametrize("Cg", [16, 6])
def test_packed_offset_mask_rows(dtype, rc, Cg, tune, monkeypatch):
    """offset = packed[..., :2GP], mask = packed[..., 2GP:3GP] with a row
    stride of 3GP (+ 5 spare elements), consumed in place."""
    if tune:
        monkeypatch.setenv("DCNV4_TUNE", tune)
    else:
        monkeypatch.delenv("DCNV4_TUNE", raising=False)
    wl = Workload("packed", 2, 11, 12, 4, Cg, (dtype,), offset_dist=("normal", 2.0), remove_center=rc, seed=23)
    x, off, m = gen.make_inputs(wl, dtype)
    G, P = wl.G, wl.P
    spare = np.zeros(off.shape[:3] + (5,), dtype=off.dtype)
    packed = np.ascontiguousarray(np.concatenate([off, m, spare], -1))
    want = ref.forward_f32(x, packed[..., :2 * G * P], packed[..., 2 * G * P:3 * G * P], dtype=dtype, **okw(wl))
    pk = gu.dev(packed, dtype)
    oview, mview = pk[..., :2 * G * P], pk[..., 2 * G * P:3 * G * P]
    gu.announce(f"packed rows {wl.describe(dtype)} remove_center={rc} row {packed.shape[-1]}")
    out = binding.forward(gu.dev(x, dtype), oview, mview, group=G, **gkw(wl))
    torch.cuda.synchronize()
    got = gu.host(out, dtype)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
    # the same values from separate dense tensors
    dense = binding.forward(gu.dev(x, dtype), gu.dev(off, dtype), gu.dev(m, dtype), **gkw(wl))
    torch.cuda.synchronize()
    assert np.array_equal(gu.host(dense, dtype).view(np.uint8), want.view(np.uint8))


# Units split over two or four lanes, with each point's coefficients computed
# by one lane of the unit and broadcast to the others (share=1) or computed by
# every lane (share=0): the same bits either way, on whole-image windows,
# bands with the fallback, and 2-D tiles (split units of two 16-byte vectors
# take tiles on wide images), with and without the centre point.
SHARED = [
    ("full_f32_4lanes", 2, 12, 13, 4, 16, 2.0, "f32", "kernel=window,split=1"),
    ("bands_f32_4lanes", 2, 60, 60, 1, 16, 8.0, "f32", "kernel=window,full=0"),
    ("bands_bf16_2lanes", 2, 60, 60, 2, 16, 6.0, "bf16", "kernel=window,full=0,split=1"),
    ("tiles_bf16_2lanes", 1, 90, 200, 2, 16, 8.0, "bf16", "kernel=window,full=0,split=1,th=16,tw=64,r=12"),
    ("full_f16_2lanes", 2, 14, 15, 2, 16, 3.0, "f16", "kernel=window,split=1"),
]


@pytest.mark.parametrize("rc", [False, True], ids=["all9", "rc"])
@pytest.mark.parametrize("case", SHARED, ids=lambda c: c[0])
def test_shared_point_coefficients_give_the_same_bits(case, rc, monkeypatch):
    name, N, H, W, G, Cg, std, dt, tune = case
    wl = Workload(name, N, H, W, G, Cg, (dt,), offset_dist=("normal", std), remove_center=rc, seed=71)
    x, off, m = gen.make_inputs(wl, dt)
    want = ref.forward_f32(x, off, m, dtype=dt, **okw(wl))
    for share in ("0", "1"):
        monkeypatch.setenv("DCNV4_TUNE", f"{tune},share={share}")
        xd, od, md = gu.dev(x, dt), gu.dev(off, dt), gu.dev(m, dt)
        plan = binding.query_plan(xd, od, md, torch.empty_like(xd), **gkw(wl))
        assert plan["kernel"] == "window" and plan["lanes_per_unit"] in (2, 4), plan
        gu.announce(f"shared coefficients {name} rc={rc} share={share} plan={plan}")
        out = binding.forward(xd, od, md, **gkw(wl))
        torch.cuda.synchronize()
        assert np.array_equal(gu.host(out, dt).view(np.uint8), want.view(np.uint8)), share
