"""GPU parity of the module forward (dcnv4_module_forward through the C ABI),
step by step: every intermediate the library stores in the workspace is
compared with the module oracle (oracle/module.py, float64) applied to the
GPU's own previous step, and the operator step with the operator's oracle
(bit for bit: same binary32 sequence on the same stored inputs).

Bounds (u = 2^-24), each plus half an ulp of the I/O type for the final
rounding of a 16-bit result:
  projection, predictor, output projection: (K + 2) u sum|terms|
      (any order of binary32 accumulation of K exact or rounded products)
  normalisation: 6 u (|xn - beta| + |mean| rstd |gamma| + |beta|)
      (binary32 mean and rstd from binary64 statistics, one subtraction,
      one product, one fused multiply-add)
  depthwise 3x3: 11 u sum|terms| (nine fused multiply-adds after the bias)
  gate: 8 u (|y| + |xn|) + u |out| (device expf within 2 ulp, then four
      rounded operations)
"""
import numpy as np
import pytest
import torch

from deformable_convolution_vision_dcnv4_amd import binding
from deformable_convolution_vision_dcnv4_amd import inputs as gen
from oracle import module as om
from oracle import ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
U = 2.0 ** -24
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
MANT = {"f32": (23, -126), "f16": (10, -14), "bf16": (7, -126)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    binding.lib()
    yield


def ulp(v, dtype):
    mant, emin = MANT[dtype]
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return 2.0 ** (np.maximum(e, emin) - mant)


def check(name, got, want, bound, dtype):
    err = np.abs(got - want)
    tol = bound + 0.5 * ulp(np.maximum(np.abs(got), np.abs(want)) + bound, dtype) + 1e-300
    worst = float(np.max(err / tol)) if err.size else 0.0
    print(f"[module] {name} {dtype}: max err {err.max():.3g}, worst err/bound {worst:.3f}", flush=True)
    assert np.all(err <= tol), f"{name}: {int(np.sum(err > tol))} of {err.size} elements beyond the bound"


def io(a, dtype):
    """float64 values rounded to the I/O type: (host array of that type, its float64 values)."""
    h = gen.to_io(a, dtype)
    return h, gen.as_f64(h, dtype)


def make_module(seed, N, H, W, Cin, G, Cg, Cout, norm, norm_groups, rc, cs, op, dtype, offset_std=1.5):
    rng = np.random.default_rng(seed)
    C = G * Cg
    P = 9 - int(rc)
    R = 3 * G * P + (G if cs else 0)
    x_h, x64 = io(rng.standard_normal((N, H, W, Cin)), dtype)
    w = {}
    w64 = {}
    w["w_in"], w64["w_in"] = io(rng.standard_normal((C, Cin)) / np.sqrt(Cin), dtype)
    w64["b_in"] = rng.standard_normal(C).astype(np.float32).astype(np.float64) * 0.1
    w64["gamma"] = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32).astype(np.float64)
    w64["beta"] = (0.1 * rng.standard_normal(C)).astype(np.float32).astype(np.float64)
    w64["w_dw"] = (rng.standard_normal((C, 3, 3)) / 3.0).astype(np.float32).astype(np.float64)
    w64["b_dw"] = (0.05 * rng.standard_normal(C)).astype(np.float32).astype(np.float64)
    # predictor rows: offsets of about offset_std pixels, weights of about 0.5, gates of about 1
    scale = np.concatenate([np.full(2 * G * P, offset_std), np.full(G * P, 0.5), np.full(R - 3 * G * P, 1.0)])
    w["w_pred"], w64["w_pred"] = io(rng.standard_normal((R, C)) * scale[:, None] / np.sqrt(C), dtype)
    w64["b_pred"] = (0.1 * rng.standard_normal(R)).astype(np.float32).astype(np.float64)
    if op:
        w["w_out"], w64["w_out"] = io(rng.standard_normal((Cout, C)) / np.sqrt(C), dtype)
        w64["b_out"] = (0.1 * rng.standard_normal(Cout)).astype(np.float32).astype(np.float64)
    dev = {}
    for k in ("w_in", "w_pred", "w_out"):
        if k in w:
            dev[k] = gu.dev(w[k], dtype)
    for k in ("b_in", "gamma", "beta", "w_dw", "b_dw", "b_pred", "b_out"):
        if k in w64:
            dev[k] = torch.from_numpy(w64[k].astype(np.float32)).cuda()
    cfg = binding.module_config(Cin=Cin, G=G, Cg=Cg, Cout=Cout if op else C, norm=norm, norm_groups=norm_groups,
                                eps=1e-5, remove_center=rc, center_scale=cs, out_proj=op, offset_scale=1.0)
    return x_h, x64, dev, w64, cfg, P, R


def region(ws, lay, key, shape, dtype, stride=None):
    """An intermediate of the workspace as a host array of the I/O type."""
    s = 4 if dtype == "f32" else 2
    n = int(np.prod(shape[:-1])) * (stride or shape[-1])
    raw = ws[lay[key]:lay[key] + n * s].cpu().numpy()
    a = raw.view({"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype])
    return a.reshape(tuple(shape[:-1]) + (stride or shape[-1],))


def norm_bound(xp, xn_ref, w64, norm, groups, eps):
    N, H, W, C = xp.shape
    if norm == binding.NORM_GROUP:
        v = xp.reshape(N, H * W, groups, C // groups)
        mean = v.mean(axis=(1, 3), keepdims=True)
        rstd = 1.0 / np.sqrt(((v - mean) ** 2).mean(axis=(1, 3), keepdims=True) + eps)
        mean = np.broadcast_to(mean, v.shape).reshape(xp.shape)
        rstd = np.broadcast_to(rstd, v.shape).reshape(xp.shape)
    else:
        mean = xp.mean(axis=-1, keepdims=True)
        rstd = 1.0 / np.sqrt(((xp - mean) ** 2).mean(axis=-1, keepdims=True) + eps)
    g, b = np.abs(w64["gamma"]), np.abs(w64["beta"])
    return 6 * U * (np.abs(xn_ref - w64["beta"]) + np.abs(mean) * rstd * g + b)


CASES = [
    # (N, H, W, Cin, G, Cg, Cout, norm, norm_groups, rc, cs, op, dtype)
    (2, 9, 11, 24, 4, 8, 20, binding.NORM_GROUP, 8, False, True, True, "f32"),
    (2, 9, 11, 24, 4, 8, 32, binding.NORM_LAYER, 1, True, True, False, "f16"),
    (2, 9, 11, 24, 4, 8, 12, binding.NORM_GROUP, 4, False, False, True, "bf16"),
    (2, 9, 11, 24, 4, 8, 32, binding.NORM_NONE, 1, False, False, False, "f16"),
    (1, 13, 7, 20, 2, 12, 28, binding.NORM_LAYER, 1, True, True, True, "bf16"),
    (3, 5, 6, 7, 3, 5, 15, binding.NORM_GROUP, 3, False, True, False, "f32"),
    # binary32 rows of 256 and 640 bytes (the projection kernel's 4- and 10-vector forms)
    (2, 6, 10, 64, 4, 16, 40, binding.NORM_GROUP, 8, False, True, True, "f32"),
    (1, 5, 9, 160, 2, 8, 16, binding.NORM_NONE, 1, False, False, True, "f32"),
    # the FlashInternImage-T stage-1 shape (batch 2, and batch 24: more row tiles
    # than projection workgroups) and the latent shape (batch 1)
    (2, 56, 56, 64, 4, 16, 64, binding.NORM_GROUP, 32, False, True, True, "f16"),
    (24, 56, 56, 64, 4, 16, 64, binding.NORM_GROUP, 32, False, True, True, "f16"),
    (1, 64, 64, 320, 8, 40, 320, binding.NORM_LAYER, 1, False, False, False, "bf16"),
]


def _id(c):
    N, H, W, Cin, G, Cg, Cout, norm, ng, rc, cs, op, dt = c
    return (f"{dt}-{N}x{H}x{W}x{Cin}-G{G}Cg{Cg}-norm{norm}" + ("-rc" if rc else "") + ("-gate" if cs else "") +
            (f"-out{Cout}" if op else ""))


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_module_forward_step_by_step(case):
    check_case(case)


def check_case(case, seed=7, offset_std=1.5):
    """Run one module configuration through the C ABI and check every step
    against the module oracle applied to the GPU's previous step."""
    N, H, W, Cin, G, Cg, Cout, norm, ng, rc, cs, op, dtype = case
    C = G * Cg
    x_h, x64, dev, w64, cfg, P, R = make_module(seed, N, H, W, Cin, G, Cg, Cout, norm, ng, rc, cs, op, dtype,
                                                offset_std=offset_std)
    gu.announce(f"module {_id(case)}")
    out, ws, lay = binding.module_forward(gu.dev(x_h, dtype), dev, cfg)
    torch.cuda.synchronize()
    shape = (N, H, W, C)
    f = lambda a: gen.as_f64(a, dtype)  # noqa: E731
    # 1. projection
    xp = f(region(ws, lay, "xp", shape, dtype))
    check("projection", xp, om.conv1x1(x64, w64["w_in"], w64["b_in"]),
          (Cin + 2) * U * om.abs_terms_conv1x1(x64, w64["w_in"], w64["b_in"]), dtype)
    # 2. normalisation
    if norm == binding.NORM_NONE:
        xn_h = region(ws, lay, "xp", shape, dtype)
    else:
        xn_h = region(ws, lay, "xn", shape, dtype)
        want = (om.group_norm(xp, ng, w64["gamma"], w64["beta"], 1e-5) if norm == binding.NORM_GROUP else
                om.layer_norm(xp, w64["gamma"], w64["beta"], 1e-5))
        check("normalisation", f(xn_h), want, norm_bound(xp, want, w64, norm, ng, 1e-5), dtype)
    xn = f(xn_h)
    # 3. depthwise 3x3, 4. predictor
    d = f(region(ws, lay, "d", shape, dtype))
    check("depthwise 3x3", d, om.dwconv3x3(xn, w64["w_dw"], w64["b_dw"]),
          11 * U * om.abs_terms_dwconv3x3(xn, w64["w_dw"], w64["b_dw"]), dtype)
    rows_h = region(ws, lay, "rows", (N, H, W, R), dtype, stride=lay["rows_stride"])
    rows = f(rows_h)[..., :R]
    check("predictor", rows, om.conv1x1(d, w64["w_pred"], w64["b_pred"]),
          (C + 2) * U * om.abs_terms_conv1x1(d, w64["w_pred"], w64["b_pred"]), dtype)
    # 5. the operator, bit for bit on the stored xn and rows
    off_v, msk_v = om.split_params(rows_h, G, P)
    y_want = ref.forward_f32(xn_h, off_v, msk_v, dtype=dtype, K=3, stride=1, pad=1, dil=1, offset_scale=1.0,
                             remove_center=rc, groups=G)
    y_h = region(ws, lay, "y", shape, dtype) if (cs or op) else gu.host(out, dtype)
    assert np.array_equal(y_h.view(np.uint8), y_want.view(np.uint8)), "operator step differs from the oracle"
    # 6. centre-feature gate, 7. output projection
    gate_and_projection(ws, lay, gu.host(out, dtype), y_h, xn, rows, w64, G, P, cs, op, dtype, stored=False)


def gate_and_projection(ws, lay, out_h, y_h, xn, rows, w64, G, P, cs, op, dtype, stored):
    """Steps 6 and 7 against the oracle applied to the stored y and xn.  With
    both steps the library may apply the gate while the projection reads its
    rows (nothing stored in between): the output is then checked against the
    oracle's gate and projection, the gate's error (its bound, plus half an
    ulp of the I/O type for the rounding of each gated value) carried through
    the projection's weights.  stored: the gated rows are in the workspace
    (the gate ran as its own kernel) and are checked as a step of their own."""
    f = lambda a: gen.as_f64(a, dtype)  # noqa: E731
    shape = y_h.shape
    C = shape[-1]
    yv = f(y_h)
    last = yv
    if cs:
        g_ref = om.centre_scale(yv, xn, rows[..., 3 * G * P:3 * G * P + G], G)
        g_bound = 8 * U * (np.abs(yv) + np.abs(xn)) + U * np.abs(g_ref)
        if not op or stored:
            g_h = region(ws, lay, "gated", shape, dtype) if op else out_h
            check("centre gate", f(g_h), g_ref, g_bound, dtype)
            last = f(g_h)
        else:
            eg = g_bound + (0.5 * ulp(np.abs(g_ref) + g_bound, dtype) if dtype != "f32" else 0.0)
            want = om.conv1x1(g_ref, w64["w_out"], w64["b_out"])
            bound = (om.conv1x1(eg, np.abs(w64["w_out"]), np.zeros_like(w64["b_out"])) +
                     (C + 2) * U * om.abs_terms_conv1x1(np.abs(g_ref) + eg, w64["w_out"], w64["b_out"]))
            check("centre gate and output projection", f(out_h), want, bound, dtype)
            return
    if op:
        check("output projection", f(out_h), om.conv1x1(last, w64["w_out"], w64["b_out"]),
              (C + 2) * U * om.abs_terms_conv1x1(last, w64["w_out"], w64["b_out"]), dtype)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_module_gate_in_its_own_kernel_when_the_output_is_unaligned(dtype):
    """An output that is not 16-byte aligned keeps the gate in its own kernel
    (the vector projection needs aligned rows): the gated rows are then in
    the workspace and checked as a step, and the projection on them."""
    N, H, W, Cin, G, Cg, Cout = 2, 9, 11, 24, 4, 16, 32
    C = G * Cg
    x_h, x64, dev, w64, cfg, P, R = make_module(13, N, H, W, Cin, G, Cg, Cout, binding.NORM_GROUP, 8, False, True,
                                                True, dtype)
    n = N * H * W * Cout
    big = torch.empty(n + 8, dtype=TDT[dtype], device="cuda")
    out = big[1:1 + n].view(N, H, W, Cout)
    assert out.data_ptr() % 16 != 0
    out, ws, lay = binding.module_forward(gu.dev(x_h, dtype), dev, cfg, out=out)
    torch.cuda.synchronize()
    shape = (N, H, W, C)
    f = lambda a: gen.as_f64(a, dtype)  # noqa: E731
    xn = f(region(ws, lay, "xn", shape, dtype))
    rows = f(region(ws, lay, "rows", (N, H, W, R), dtype, stride=lay["rows_stride"]))[..., :R]
    y_h = region(ws, lay, "y", shape, dtype)
    gate_and_projection(ws, lay, gu.host(out, dtype), y_h, xn, rows, w64, G, P, True, True, dtype, stored=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_module_with_identity_predictor_returns_the_normalised_input(dtype):
    """Predictor weights zero and biases that give zero offsets and a weight
    of one on the centre point only: the operator copies xn, bit for bit (the
    packed rows reach the operator at the right offsets and stride)."""
    N, H, W, Cin, G, Cg = 2, 6, 7, 16, 2, 8
    x_h, x64, dev, w64, cfg, P, R = make_module(11, N, H, W, Cin, G, Cg, G * Cg, binding.NORM_LAYER, 1, False,
                                                False, False, dtype)
    dev["w_pred"].zero_()
    b = np.zeros(R, dtype=np.float32)
    for g in range(G):
        b[2 * G * P + g * P + 4] = 1.0
    dev["b_pred"] = torch.from_numpy(b).cuda()
    out, ws, lay = binding.module_forward(gu.dev(x_h, dtype), dev, cfg)
    torch.cuda.synchronize()
    xn_h = region(ws, lay, "xn", (N, H, W, G * Cg), dtype)
    assert np.array_equal(gu.host(out, dtype).view(np.uint8), xn_h.view(np.uint8))


def test_module_is_reproducible_and_fills_a_given_workspace():
    N, H, W, Cin, G, Cg = 2, 12, 10, 32, 4, 8
    x_h, x64, dev, w64, cfg, P, R = make_module(13, N, H, W, Cin, G, Cg, 24, binding.NORM_GROUP, 8, True, True,
                                                True, "f16")
    x = gu.dev(x_h, "f16")
    lay = binding.module_layout(N, H, W, cfg, torch.float16)
    ws = torch.full((lay["total"] + 4096,), 0x7F, dtype=torch.uint8, device="cuda")
    o1, _, _ = binding.module_forward(x, dev, cfg, workspace=ws)
    o1 = o1.clone()
    ws.fill_(0xFF)
    o2, _, _ = binding.module_forward(x, dev, cfg, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # the bytes past the layout's total are untouched
    assert torch.all(ws[lay["total"]:] == 0xFF)
