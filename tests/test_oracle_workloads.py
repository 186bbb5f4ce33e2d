"""The two oracle modes agree on every workload's inputs (CPU only).

The binary32 sequence must sit within the forward-error bound of the plain
double-precision definition, and the I/O-typed runs within half an output ulp
more.  Batch is cut to keep the CPU suite short; shapes are the workloads'.
"""
import dataclasses

import numpy as np
import pytest

from deformable_convolution_vision_dcnv4_amd import inputs as gen
from deformable_convolution_vision_dcnv4_amd.workloads import WORKLOADS
from oracle import ref
from tests import helpers as H

CASES = [(name, dt) for name, wl in WORKLOADS.items() for dt in wl.dtypes]


@pytest.mark.parametrize("name,dtype", CASES)
def test_f32_sequence_within_bound_of_definition(name, dtype):
    wl = WORKLOADS[name]
    wl = dataclasses.replace(wl, N=min(wl.N, 2))
    x, off, m = gen.make_inputs(wl, dtype)
    kw = dict(K=wl.K, stride=wl.stride, pad=wl.pad, dil=wl.dil, offset_scale=wl.offset_scale)
    got = ref.to_f32(ref.forward_f32(x, off, m, dtype=dtype, **kw), dtype).astype(np.float64)
    x64, o64, m64 = (gen.as_f64(a, dtype) for a in (x, off, m))
    exact = ref.forward_f64(x64, o64, m64, **kw)
    bound = H.f32_bound(x64, o64, m64, wl.K, wl.stride, wl.pad, wl.dil, scale=wl.offset_scale)
    if dtype != "f32":
        half_ulp = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
        bound = bound * (1 + half_ulp) + np.abs(exact) * half_ulp * (1 + 1e-6) + 2.0 ** -133
    err = np.abs(got - exact)
    assert np.all(err <= bound), float(np.max(err - bound))
    # and the error is far from the bound's scale for most outputs
    rms = float(np.sqrt(np.mean(exact ** 2)))
    assert rms > 0.1
