"""Shared pieces of the GPU tests: host<->device transfer of I/O-typed arrays
and the parity comparison (tolerances of the operator's contract)."""
import sys

import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# max |gpu - oracle|: fp32 absolute; fp16/bf16 relative to the oracle output's RMS
TOL_F32_ABS = 1e-5
TOL_16_REL_RMS = 2e-3


def dev(a, dtype, device="cuda"):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def host(t, dtype):
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen(a, dtype):
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32)


def compare(got, want, dtype, label=""):
    """Assert the contract's tolerance; return (max_abs, rms, n_bit_mismatch)."""
    g, w = widen(got, dtype).astype(np.float64), widen(want, dtype).astype(np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    finite = np.isfinite(w)
    assert np.array_equal(np.isfinite(g), finite), f"{label}: non-finite pattern differs"
    err = np.abs(g[finite] - w[finite])
    max_abs = float(err.max()) if err.size else 0.0
    rms = float(np.sqrt(np.mean(w[finite] ** 2))) if err.size else 0.0
    bits_g = got.view(np.uint32 if dtype == "f32" else np.uint16)
    bits_w = want.view(np.uint32 if dtype == "f32" else np.uint16)
    mism = int(np.count_nonzero((bits_g != bits_w) & finite & ~((g == 0) & (w == 0))))
    print(f"[parity] {label} dtype={dtype} n={w.size} max_abs={max_abs:.3e} rms={rms:.3e} "
          f"bit_mismatch={mism}", flush=True)
    if dtype == "f32":
        assert max_abs <= TOL_F32_ABS, f"{label}: max abs err {max_abs} > {TOL_F32_ABS}"
    else:
        assert max_abs <= TOL_16_REL_RMS * rms, f"{label}: max abs err {max_abs} > 2e-3*RMS ({rms})"
    return max_abs, rms, mism


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()
