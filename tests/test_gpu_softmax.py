"""GPU parity of the DCNv3-style aggregation (dcnv4_forward_softmax).

Every case runs on both kernel families (the window family where the
shape allows it, else the direct kernel again), which must agree bit for bit.

Reference: the oracle's binary32 operation sequence fed with the oracle's
softmax weights (double precision, rounded to binary32).  The GPU computes
the weights in binary32 with the device's expf: each weight then differs
from the reference weight by at most (2 * max|m - max m| + P + 8) * u
relatively (the exponent's argument, expf, the P-term sum and the division,
on either side), u = 2^-24.  The outputs differ by at most that times
A = sum |w * bilinear weight * x| (computed in double), and a 16-bit output
by at most one unit in the last place more (a final rounding that lands on
the other side of a tie).
"""
import numpy as np
import pytest
import torch

from deformable_convolution_vision_dcnv4_amd import binding
from deformable_convolution_vision_dcnv4_amd import inputs as gen
from deformable_convolution_vision_dcnv4_amd.workloads import WORKLOADS, Workload
from oracle import ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    binding.lib()
    yield


def ulp16(v, dtype):
    mbits = 10 if dtype == "f16" else 7
    emin = -14 if dtype == "f16" else -126
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** emin)))
    return 2.0 ** (e - mbits)


def check(wl, dtype, monkeypatch):
    x, off, m = gen.make_inputs(wl, dtype)
    kw = dict(K=wl.K, stride=wl.stride, pad=wl.pad, dil=wl.dil, offset_scale=wl.offset_scale,
              remove_center=wl.remove_center)
    x32, o32, m32 = (ref.to_f32(a, dtype) for a in (x, off, m))
    G, P = wl.G, wl.P
    w64 = ref.softmax_weights(m32.astype(np.float64), groups=G, P=P)
    want = ref.forward_f32(x32, o32, w64.astype(np.float32), dtype="f32", **kw).astype(np.float64)
    A = ref.forward_f64(np.abs(x32.astype(np.float64)), o32.astype(np.float64), w64, **kw)
    dm = np.max(np.abs(m32.reshape(*m32.shape[:3], G, P) - m32.reshape(*m32.shape[:3], G, P).max(-1, keepdims=True)))
    tol = (2 * dm + P + 8) * U * A
    if dtype != "f32":
        tol = tol + ulp16(want, dtype)
    xd, od, md = gu.dev(x, dtype), gu.dev(off, dtype), gu.dev(m, dtype)
    outs = {}
    # both kernel families (the window family where the shape allows it): the
    # same weights and operation sequence, so the same bits
    for fam in ("direct", "window"):
        monkeypatch.setenv("DCNV4_TUNE", f"kernel={fam}")
        gu.announce(f"softmax {wl.describe(dtype)} remove_center={wl.remove_center} kernel={fam}")
        out = binding.forward(xd, od, md, kernel_size=wl.K, stride=wl.stride, pad=wl.pad, dilation=wl.dil,
                              offset_scale=wl.offset_scale, remove_center=wl.remove_center, softmax=True)
        torch.cuda.synchronize()
        outs[fam] = gu.host(out, dtype)
        got = ref.to_f32(outs[fam], dtype).astype(np.float64)
        err = np.abs(got - want)
        print(f"  {fam}: max err {err.max():.3g}, max tol {tol.max():.3g}")
        assert np.all(err <= tol), f"{fam}: {np.sum(err > tol)} outputs beyond the bound"
    monkeypatch.delenv("DCNV4_TUNE", raising=False)
    assert np.array_equal(outs["direct"].view(np.uint8), outs["window"].view(np.uint8)), \
        "the two kernel families disagree"


CASES = [(Workload("sm", 2, 11, 13, 4, Cg, (dt,), offset_dist=("normal", 2.0), mask_dist=("normal", 2.0),
                   remove_center=rc, seed=61), dt)
         for dt in ("f32", "f16", "bf16") for Cg in (16, 6) for rc in (False, True)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[1]}-Cg{c[0].Cg}{'-rc' if c[0].remove_center else ''}")
def test_softmax_variant_matches_oracle(case, monkeypatch):
    check(*case, monkeypatch)


@pytest.mark.parametrize("name,dtype", [("fiit_stage1", "f16"), ("fiit_stage1", "f32"), ("fiit_stage3", "f16"),
                                        ("hires", "bf16"), ("sd_latent", "bf16"), ("tiny", "f32")])
def test_softmax_variant_workloads(name, dtype, monkeypatch):
    """Every workload at full size: the whole-image window, bands of units
    split over lanes with shared coefficients (stage-1 f32), tiles with the
    global fallback (hires) and bands of five-vector units (latent)."""
    check(WORKLOADS[name], dtype, monkeypatch)


def test_softmax_of_huge_weights_is_finite_and_box_mean_for_equal_weights():
    wl = Workload("smbig", 1, 8, 9, 2, 8, ("f32",), seed=62)
    x, off, m = gen.make_inputs(wl, "f32")
    big = np.full_like(m, 1000.0)
    zero = np.zeros_like(off)
    out = binding.forward(gu.dev(x, "f32"), gu.dev(zero, "f32"), gu.dev(big, "f32"), softmax=True)
    torch.cuda.synchronize()
    got = gu.host(out, "f32").astype(np.float64)
    assert np.all(np.isfinite(got))
    xp = np.pad(x.astype(np.float64), ((0, 0), (1, 1), (1, 1), (0, 0)))
    box = sum(xp[:, i:i + 8, j:j + 9] for i in range(3) for j in range(3)) / 9.0
    np.testing.assert_allclose(got, box, rtol=0, atol=64 * U * np.abs(x).max())
