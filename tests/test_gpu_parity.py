"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every comparison is element by element on the same seeded inputs.  The
contract: bit-exact for integer offsets in fp32; otherwise max abs error
<= 1e-5 (fp32) and <= 2e-3 * RMS(output) (fp16/bf16).  Because the kernels
follow the oracle's binary32 operation sequence, every case is also checked
for bit-identity.
"""
import dataclasses

import numpy as np
import pytest
import torch

from deformable_convolution_vision_dcnv4_amd import binding
from deformable_convolution_vision_dcnv4_amd import inputs as gen
from deformable_convolution_vision_dcnv4_amd.workloads import SENSITIVITY, WORKLOADS, Workload
from oracle import ref
from tests import gpu_util as gu
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    binding.lib()   # fail loudly if the HIP library is missing
    yield


@pytest.fixture(params=["auto", "window"], autouse=True)
def family(request, monkeypatch):
    """Every test twice: with the planner's own choice (small batches take the
    direct kernel) and with the window family forced wherever it applies
    (DCNV4_TUNE=kernel=window), so both families meet every case."""
    if request.param == "window":
        monkeypatch.setenv("DCNV4_TUNE", "kernel=window")
    else:
        monkeypatch.delenv("DCNV4_TUNE", raising=False)
    return request.param


def run_gpu(x, off, m, dtype, wl=None, **kw):
    xs, os_, ms = gu.dev(x, dtype), gu.dev(off, dtype), gu.dev(m, dtype)
    out = binding.forward(xs, os_, ms, **kw)
    torch.cuda.synchronize()
    return gu.host(out, dtype)


def kw_of(wl):
    return dict(kernel_size=wl.K, stride=wl.stride, pad=wl.pad, dilation=wl.dil,
                offset_scale=wl.offset_scale, remove_center=wl.remove_center)


def okw_of(wl):
    return dict(K=wl.K, stride=wl.stride, pad=wl.pad, dil=wl.dil, offset_scale=wl.offset_scale,
                remove_center=wl.remove_center)


CASES = [(name, dt) for name, wl in WORKLOADS.items() for dt in wl.dtypes]


@pytest.mark.parametrize("name,dtype", CASES)
def test_workload_parity_full_size(name, dtype):
    """Every workload at its full size, in the launch configuration the bench uses."""
    wl = WORKLOADS[name]
    gu.announce(f"workload {wl.describe(dtype)} seed {wl.seed}")
    x, off, m = gen.make_inputs(wl, dtype)
    want = ref.forward_f32(x, off, m, dtype=dtype, **okw_of(wl))
    got = run_gpu(x, off, m, dtype, **kw_of(wl))
    _, _, mism = gu.compare(got, want, dtype, label=name)
    assert mism == 0, f"{mism} outputs differ in bits from the oracle's binary32 sequence"


@pytest.mark.parametrize("name", list(SENSITIVITY))
def test_sensitivity_inputs_full_size(name):
    """The smooth-offset sensitivity input at full size, as the bench times it."""
    wl = SENSITIVITY[name]
    for dtype in wl.dtypes:
        gu.announce(f"sensitivity {wl.describe(dtype)} smooth {wl.offset_smooth} seed {wl.seed}")
        x, off, m = gen.make_inputs(wl, dtype)
        want = ref.forward_f32(x, off, m, dtype=dtype, **okw_of(wl))
        got = run_gpu(x, off, m, dtype, **kw_of(wl))
        _, _, mism = gu.compare(got, want, dtype, label=name)
        assert mism == 0, f"{mism} outputs differ in bits from the oracle's binary32 sequence"


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_integer_offsets_bit_exact_fp32(name):
    """Integer offsets, fp32: exact shifted gathers, bit-identical."""
    wl = WORKLOADS[name]
    gu.announce(f"integer offsets fp32 {wl.describe('f32')}")
    x, off, m = gen.make_inputs(wl, "f32", integer_offsets=True)
    want = ref.forward_f32(x, off, m, dtype="f32", **okw_of(wl))
    got = run_gpu(x, off, m, "f32", **kw_of(wl))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_matches_float64_definition_within_bound():
    wl = dataclasses.replace(WORKLOADS["fiit_stage1"], N=2)
    x, off, m = gen.make_inputs(wl, "f32")
    got = run_gpu(x, off, m, "f32", **kw_of(wl)).astype(np.float64)
    x64, o64, m64 = (a.astype(np.float64) for a in (x, off, m))
    exact = ref.forward_f64(x64, o64, m64, **okw_of(wl))
    bound = H.f32_bound(x64, o64, m64, wl.K, wl.stride, wl.pad, wl.dil)
    assert np.all(np.abs(got - exact) <= bound)


SWEEP = []
for Cg in (1, 2, 3, 4, 8, 16, 24, 32, 40, 64, 128):
    SWEEP.append(dict(Cg=Cg, G=2, K=3, s=1, p=1, d=1, scale=1.0))
for K, s, p, d in ((1, 1, 0, 1), (5, 1, 2, 1), (3, 2, 1, 1), (3, 1, 2, 2), (3, 2, 0, 2), (5, 2, 1, 2),
                   (2, 1, 0, 1), (3, 3, 1, 1), (7, 1, 3, 1)):
    SWEEP.append(dict(Cg=16, G=3, K=K, s=s, p=p, d=d, scale=1.0))
for scale in (0.0, 0.5, 2.0, -1.25):
    SWEEP.append(dict(Cg=8, G=4, K=3, s=1, p=1, d=1, scale=scale))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "Cg{Cg}_G{G}_K{K}_s{s}_p{p}_d{d}_sc{scale}".format(**c))
def test_shape_sweep_bit_exact(case, dtype):
    wl = Workload("sweep", 2, 13, 11, case["G"], case["Cg"], (dtype,), offset_dist=("normal", 2.0),
                  mask_dist=("normal", 0.7), K=case["K"], stride=case["s"], pad=case["p"],
                  dil=case["d"], offset_scale=case["scale"], seed=7)
    gu.announce(f"sweep {wl.describe(dtype)} scale {wl.offset_scale}")
    x, off, m = gen.make_inputs(wl, dtype)
    want = ref.forward_f32(x, off, m, dtype=dtype, **okw_of(wl))
    got = run_gpu(x, off, m, dtype, **kw_of(wl))
    gu.compare(got, want, dtype, label="sweep")
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shift", [1, 2, 3, 4])
def test_misaligned_pointers_same_bits(dtype, shift):
    """Base pointers shifted by whole elements force narrower vectors; the
    result must not change."""
    wl = Workload("misaligned", 2, 9, 10, 4, 16, (dtype,), offset_dist=("normal", 1.5), seed=3)
    x, off, m = gen.make_inputs(wl, dtype)
    want = ref.forward_f32(x, off, m, dtype=dtype, **okw_of(wl))
    xs = gu.dev(x, dtype)
    base = torch.empty(xs.numel() + 8, dtype=xs.dtype, device="cuda")
    xv = base[shift:shift + xs.numel()].view(xs.shape)
    xv.copy_(xs)
    obase = torch.empty(xs.numel() + 8, dtype=xs.dtype, device="cuda")
    ov = obase[shift:shift + xs.numel()].view(xs.shape)
    plan = binding.query_plan(xv, gu.dev(off, dtype), gu.dev(m, dtype), ov, **kw_of(wl))
    gu.announce(f"misaligned shift {shift} {dtype} plan {plan}")
    binding.forward(xv, gu.dev(off, dtype), gu.dev(m, dtype), out=ov, **kw_of(wl))
    torch.cuda.synchronize()
    got = gu.host(ov, dtype)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_non_default_stream_and_determinism():
    wl = WORKLOADS["fiit_stage3"]
    x, off, m = gen.make_inputs(wl, "f16")
    xs, os_, ms = gu.dev(x, "f16"), gu.dev(off, "f16"), gu.dev(m, "f16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = binding.forward(xs, os_, ms)
    b = binding.forward(xs, os_, ms, stream=s)
    s.synchronize()
    c = binding.forward(xs, os_, ms)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_raw_entry_point():
    """dcnv4_forward with raw pointers, exactly the plain ABI signature."""
    wl = WORKLOADS["tiny"]
    x, off, m = gen.make_inputs(wl, "f32")
    xs, os_, ms = gu.dev(x, "f32"), gu.dev(off, "f32"), gu.dev(m, "f32")
    out = torch.full_like(xs, float("nan"))
    binding.forward_raw(xs.data_ptr(), os_.data_ptr(), ms.data_ptr(), out.data_ptr(), wl.N, wl.H, wl.W,
                        wl.G, wl.Cg, 3, 1, 1, 1, 1.0, binding.F32, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = ref.forward_f32(x, off, m, dtype="f32")
    assert np.array_equal(gu.host(out, "f32").view(np.uint32), want.view(np.uint32))


def test_empty_batch_and_single_pixel():
    xs = torch.zeros((0, 5, 5, 8), device="cuda")
    out = binding.forward(xs, torch.zeros((0, 5, 5, 36), device="cuda"), torch.zeros((0, 5, 5, 18), device="cuda"))
    assert out.shape == (0, 5, 5, 8)
    wl = Workload("one", 1, 1, 1, 2, 4, ("f32",), offset_dist=("normal", 0.5), seed=5)
    x, off, m = gen.make_inputs(wl, "f32")
    want = ref.forward_f32(x, off, m, dtype="f32")
    got = run_gpu(x, off, m, "f32")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_all_outside_and_nan_offsets_give_zero():
    wl = Workload("oob", 2, 6, 7, 2, 8, ("f32",), seed=9)
    x, off, m = gen.make_inputs(wl, "f32")
    for fill in (100.0, -100.0, float("nan"), 1e30):
        o = np.full_like(off, fill)
        got = run_gpu(x, o, m, "f32")
        assert np.array_equal(got, np.zeros_like(got)), fill


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_io_rounding_matches_fp32_path(dtype):
    """Inputs representable in the I/O type: the 16-bit run equals the fp32 run
    rounded once (checked on the GPU outputs themselves)."""
    wl = Workload("xdtype", 2, 12, 12, 4, 16, (dtype,), offset_dist=("normal", 2.0), seed=11)
    x, off, m = gen.make_inputs(wl, dtype)
    got16 = run_gpu(x, off, m, dtype)
    got32 = run_gpu(ref.to_f32(x, dtype), ref.to_f32(off, dtype), ref.to_f32(m, dtype), "f32")
    assert np.array_equal(got16.view(np.uint16), ref.from_f32(got32, dtype).view(np.uint16))
