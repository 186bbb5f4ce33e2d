"""The module forward's no-allocation entry point (dcnv4_module_forward_noalloc,
for callers that cannot allocate device memory) through the C ABI: its
output equals dcnv4_module_forward's with a caller workspace, bit for bit (the
same kernels, so the same binary32 sequence), on two calls in a row, the
second with a smaller input; problems beyond the scratch array are rejected
before any HIP call."""
import ctypes

import numpy as np
import pytest
import torch

from deformable_convolution_vision_dcnv4_amd import binding
from tests import gpu_util as gu
from tests.test_gpu_module import make_module

pytestmark = pytest.mark.gpu


def _noalloc(x, dev, cfg, out):
    w = binding.ModuleWeights()
    for name, _ in w._fields_:
        t = dev.get(name)
        if t is not None:
            setattr(w, name, t.data_ptr())
    N, H, W, _ = x.shape
    st = binding.lib().dcnv4_module_forward_noalloc(x.data_ptr(), ctypes.byref(w), out.data_ptr(), N, H, W,
                                                   ctypes.byref(cfg), binding._DTYPE_CODE[x.dtype],
                                                   torch.cuda.current_stream().cuda_stream)
    return st


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_noalloc_module_equals_workspace_module_twice(dtype):
    assert torch.cuda.is_available()
    # (N, H, W) of the two calls: the second smaller; the same weights
    shapes = [(3, 28, 30), (1, 9, 11)]
    Cin, G, Cg, Cout = 32, 4, 8, 24
    x_h, _, dev, _, cfg, _, _ = make_module(17, 3, 28, 30, Cin, G, Cg, Cout, binding.NORM_GROUP, 8, False, True,
                                           True, dtype)
    xs = gu.dev(x_h, dtype)
    for i, (N, H, W) in enumerate(shapes):
        x = xs[:N, :H, :W].contiguous()
        lay = binding.module_layout(N, H, W, cfg, x.dtype)
        assert lay["total"] <= binding.MODULE_SCRATCH_BYTES
        gu.announce(f"no-alloc module call {i}: {N}x{H}x{W} {dtype}")
        want, _, _ = binding.module_forward(x, dev, cfg)
        got = torch.full_like(want, float("nan"))
        assert _noalloc(x, dev, cfg, got) == 0, binding.last_error()
        torch.cuda.synchronize()
        a, b = gu.host(got, dtype), gu.host(want, dtype)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"call {i} differs"


def test_noalloc_module_rejects_problems_beyond_its_scratch():
    cfg = binding.module_config(Cin=64, G=4, Cg=16, Cout=64, norm=binding.NORM_GROUP, norm_groups=32)
    lay = binding.module_layout(64, 56, 56, cfg, torch.float16)
    assert lay["total"] > binding.MODULE_SCRATCH_BYTES
    w = binding.ModuleWeights()
    for i, (name, _) in enumerate(w._fields_):
        setattr(w, name, 0x30000000 + i * 0x100000)
    st = binding.lib().dcnv4_module_forward_noalloc(0x10000000, ctypes.byref(w), 0x20000000, 64, 56, 56,
                                                   ctypes.byref(cfg), 1, None)
    assert st == 6 and "no-allocation" in binding.last_error()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_noalloc_module_captured_in_a_graph_replays_the_eager_result(dtype):
    """The callers it is for: code under HIP graph capture.  The entry point
    is captured once (its scratch address was looked up by an eager call
    before), then the graph is replayed several times with new input values
    copied in between and eager work and synchronisations around the
    replays; every replay must equal the workspace entry point's eager
    result on the same input, bit for bit."""
    N, H, W, Cin, G, Cg, Cout = 2, 12, 14, 32, 4, 8, 24
    x_h, _, dev, _, cfg, _, _ = make_module(23, N, H, W, Cin, G, Cg, Cout, binding.NORM_GROUP, 8, False, True,
                                           True, dtype)
    x = gu.dev(x_h, dtype)
    out = torch.empty((N, H, W, Cout), dtype=x.dtype, device=x.device)
    assert _noalloc(x, dev, cfg, out) == 0, binding.last_error()   # eager call first
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = _noalloc(x, dev, cfg, out)
    assert st == 0, binding.last_error()
    torch.cuda.synchronize()
    gen_ = torch.Generator(device="cpu").manual_seed(5)
    for i in range(4):
        # new input values in the captured buffer, eager work around the replay
        x.copy_((torch.randn(x.shape, generator=gen_) * (1 + i)).to(x.dtype))
        want, _, _ = binding.module_forward(x, dev, cfg)
        torch.cuda.synchronize()
        gu.announce(f"graph replay {i} {dtype}")
        g.replay()
        torch.cuda.synchronize()
        a, b = gu.host(out, dtype), gu.host(want, dtype)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {i} differs from the eager result"
