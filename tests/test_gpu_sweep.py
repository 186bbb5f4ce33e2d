"""Randomised GPU parity sweep with a fixed seed: small shapes over all
dtypes, K in {1, 3, 5}, strides, pads, dilations, remove_center, offsets of
0.5 to 8 pixels' spread and offset scales.  The forward must equal the
oracle's binary32 sequence bit for bit, both with the planner's own choice
and with the window family forced (DCNV4_TUNE=kernel=window); on every other
case the backward must lie within the oracle's rounding bounds (as in
test_gpu_backward, with a generous allowance for the fixed-point quantum)."""
import random

import numpy as np
import pytest
import torch

from deformable_convolution_vision_dcnv4_amd import binding
from deformable_convolution_vision_dcnv4_amd import inputs as gen
from deformable_convolution_vision_dcnv4_amd.workloads import Workload
from oracle import ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _cases(seed, n):
    rng = random.Random(seed)
    out = []
    for case in range(n):
        while True:
            K = rng.choice([3, 3, 3, 1, 5])
            s = rng.choice([1, 1, 2])
            d = rng.choice([1, 1, 2])
            p = rng.randint(0, 3)
            H, W = rng.randint(1, 90), rng.randint(1, 90)
            Ho = (H + 2 * p - d * (K - 1) - 1) // s + 1
            Wo = (W + 2 * p - d * (K - 1) - 1) // s + 1
            if Ho >= 1 and Wo >= 1:
                break
        N = rng.choice([1, 1, 2, 3, 8, 17])
        G = rng.choice([1, 2, 4, 8])
        Cg = rng.choice([2, 4, 6, 8, 16, 16, 24, 32, 40])
        dt = rng.choice(["f32", "f16", "bf16"])
        rc = K > 1 and rng.random() < 0.3
        std = rng.choice([0.5, 2.0, 8.0])
        sc = rng.choice([0.5, 1.0, 1.7])
        if N * H * W * G * Cg > 3_000_000:
            N = 1
        out.append((case, Workload("sweep", N, H, W, G, Cg, (dt,), offset_dist=("normal", std), K=K, stride=s,
                                   pad=p, dil=d, offset_scale=sc, remove_center=rc, seed=1000 + case), dt))
    return out


CASES = _cases(21, 40)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    binding.lib()
    yield


def _f64(a, dt):
    return ref.to_f32(a, dt).astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[2]}-{c[1].N}x{c[1].H}x{c[1].W}-G{c[1].G}"
                                                      f"-Cg{c[1].Cg}-K{c[1].K}s{c[1].stride}p{c[1].pad}d{c[1].dil}")
def test_random_shape(case, monkeypatch):
    idx, wl, dt = case
    x, off, m = gen.make_inputs(wl, dt)
    okw = dict(K=wl.K, stride=wl.stride, pad=wl.pad, dil=wl.dil, offset_scale=wl.offset_scale,
               remove_center=wl.remove_center)
    gkw = dict(kernel_size=wl.K, stride=wl.stride, pad=wl.pad, dilation=wl.dil, offset_scale=wl.offset_scale,
               remove_center=wl.remove_center)
    want = ref.forward_f32(x, off, m, dtype=dt, **okw)
    for tune in ("", "kernel=window"):
        if tune:
            monkeypatch.setenv("DCNV4_TUNE", tune)
        else:
            monkeypatch.delenv("DCNV4_TUNE", raising=False)
        gu.announce(f"sweep {idx} {wl.describe(dt)} rc={wl.remove_center} tune={tune!r}")
        out = binding.forward(gu.dev(x, dt), gu.dev(off, dt), gu.dev(m, dt), **gkw)
        torch.cuda.synchronize()
        got = gu.host(out, dt)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), tune
    monkeypatch.delenv("DCNV4_TUNE", raising=False)
    if idx % 2:
        return
    Ho, Wo = wl.out_hw()
    go = gen.make_inputs(Workload("g", wl.N, Ho, Wo, wl.G, wl.Cg, (dt,), seed=2000 + idx), dt)[0]
    gx_ref, goff_ref, gm_ref, b = ref.backward_f64(_f64(x, dt), _f64(off, dt), _f64(m, dt), _f64(go, dt),
                                                   bounds=True, f32_positions=True, **okw)
    gu.announce(f"sweep {idx} backward")
    gx, goff, gm = binding.backward(*(gu.dev(a, dt) for a in (x, off, m, go)), **gkw)
    torch.cuda.synchronize()
    gx, goff, gm = (t.cpu().numpy().astype(np.float64) for t in (gx, goff, gm))
    mm = float(np.abs(ref.to_f32(m, dt)).max())
    mg = float(np.abs(ref.to_f32(go, dt)).max())
    # the fixed-point quantum 2^-(F+1) is below max|m| * max|g| * 2^-30 for any image of these sizes
    tol_x = (b["cnt_x"] + 6) * U * b["abs_x"] + b["cnt_x"] * mm * mg * 2.0 ** -30 + 1e-300
    tol_m = (4 * wl.Cg + 8) * U * b["abs_mask"] + 1e-300
    tol_o = (4 * wl.Cg + 10) * U * b["abs_offset"] + 1e-300
    assert np.all(np.abs(gx - gx_ref) <= tol_x)
    assert np.all(np.abs(gm - gm_ref) <= tol_m)
    assert np.all(np.abs(goff - goff_ref) <= tol_o)
