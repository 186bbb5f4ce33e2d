"""Backward parity at the full sizes of the benchmarked workloads (the
shapes whose backward times are reported), in both plan modes: the
planner's own choice and the whole-image kernels kept wherever they fit
(DCNV4_BWD_FILL=0).  The oracle's gradients are computed once per workload
and compared with both GPU runs; bounds as in test_gpu_backward."""
import pytest
import torch

from deformable_convolution_vision_dcnv4_amd import binding
from deformable_convolution_vision_dcnv4_amd.workloads import WORKLOADS
from tests import gpu_util as gu
from tests.test_gpu_backward import check, reference

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    binding.lib()
    yield


@pytest.mark.parametrize("name,dtype", [("fiit_stage1", "f16"), ("fiit_stage1", "f32"), ("hires", "bf16"),
                                        ("sd_latent", "bf16")])
def test_backward_full_size_workload(name, dtype, monkeypatch):
    wl = WORKLOADS[name]
    gu.announce(f"oracle backward {wl.describe(dtype)}")
    refs = reference(wl, dtype)
    for mode in ("fill", "whole"):
        if mode == "whole":
            monkeypatch.setenv("DCNV4_BWD_FILL", "0")
        else:
            monkeypatch.delenv("DCNV4_BWD_FILL", raising=False)
        gu.announce(f"backward {wl.describe(dtype)} plan mode {mode}")
        check(wl, dtype, refs=refs)
