"""The pins bite: each plausible mistake, planted in a COPY of the oracle
source on the CPU, must make the pin suite fail.  (The real oracle is never
modified; the mutated copies live in a temporary directory.)"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dcnv4_oracle.c")

MUTATIONS = {
    "trunc_not_floor": ("const float fx = floorf(px), fy = floorf(py);",
                        "const float fx = truncf(px), fy = truncf(py);"),
    "planes_swapped": ("const float dx = dxs[k], dy = dys[k], m = ms[k];",
                       "const float dx = dys[k], dy = dxs[k], m = ms[k];"),
    "corner_dropped": ("for (int b = 0; b < 2; ++b) {\n                        const int yy",
                       "for (int b = 0; b < 1; ++b) {\n                        const int yy"),
    "weights_swapped": ("{ { mhy * hx, mhy * lx }, { mly * hx, mly * lx } }",
                        "{ { mhy * lx, mhy * hx }, { mly * hx, mly * lx } }"),
    "pad_sign": ("(float)(wo * stride - pad + j * dil)", "(float)(wo * stride + pad + j * dil)"),
    "column_major_points": ("(float)(wo * stride - pad + j * dil));\n                const float py = fmaf(dy, offset_scale, (float)(ho * stride - pad + i * dil))",
                            "(float)(wo * stride - pad + i * dil));\n                const float py = fmaf(dy, offset_scale, (float)(ho * stride - pad + j * dil))"),
    "lost_negative_band": ("if (!(px > -1.0f && px < (float)W", "if (!(px >= 0.0f && px < (float)W"),
    "abs_weights": ("const float mhy = m * hy, mly = m * ly;", "const float mhy = fabsf(m) * hy, mly = fabsf(m) * ly;"),
    "scale_ignored": ("const float px = fmaf(dx, offset_scale,", "const float px = fmaf(dx, 1.0f,"),
    "dilation_ignored": ("(float)(ho * stride - pad + i * dil)", "(float)(ho * stride - pad + i)"),
    "edge_clamp_not_zero": (
        "if (yy >= 0 && yy < H && xx >= 0 && xx < W)\n"
        "                            v = xf[(((int64_t)n * H + yy) * W + xx)",
        "if (1)\n"
        "                            v = xf[(((int64_t)n * H + (yy < 0 ? 0 : yy >= H ? H - 1 : yy)) * W"
        " + (xx < 0 ? 0 : xx >= W ? W - 1 : xx))"),
    "round_toward_zero": ("double q = nearbyint(ldexp(a, mbits - e));", "double q = floor(ldexp(a, mbits - e));"),
    "f64_one_axis_weight": ("const double wgt = (1.0 - fabs(py - qy)) * (1.0 - fabs(px - qx));",
                            "const double wgt = (1.0 - fabs(py - qy));"),
    "f64_planes_swapped": ("const double dx = offset[pix * s.off_stride + (int64_t)g * 2 * s.P + k];",
                           "const double dx = offset[pix * s.off_stride + (int64_t)g * 2 * s.P + s.P + k];"),
    "bwd_dtri_sign": ("if (t >= 0.0 && t < 1.0) return -1.0;", "if (t >= 0.0 && t < 1.0) return 1.0;"),
    "bwd_offset_mask_factor_dropped": ("gox[k] = offset_scale * m * d_px;", "gox[k] = offset_scale * d_px;"),
    "bwd_offset_planes_swapped": ("gox[k] = offset_scale * m * d_px;", "gox[k] = offset_scale * m * d_py;"),
    "bwd_scale_dropped": ("gox[s.P + k] = offset_scale * m * d_py;", "gox[s.P + k] = m * d_py;"),
    "bwd_grad_x_one_axis": ("grad_x[q + c] += m * ty * tx * go[c];", "grad_x[q + c] += m * ty * go[c];"),
    "bwd_grad_mask_abs": ("d_m += go[c] * ty * tx * f;", "d_m += fabs(go[c]) * ty * tx * f;"),
    "bwd_bound_count_inflated": ("if (cnt_x) cnt_x[q + c] += 1.0;", "if (cnt_x) cnt_x[q + c] += 2.0;"),
    "bwd_bound_x_weight_dropped": ("if (abs_x) abs_x[q + c] += fabs(m * ty * tx * go[c]);",
                                   "if (abs_x) abs_x[q + c] += fabs(ty * tx * go[c]);"),
    "bwd_bound_mask_one_axis": ("a_m += fabs(go[c] * ty * tx * f);", "a_m += fabs(go[c] * ty * f);"),
    "bwd_bound_offset_weight_dropped": ("fabs(offset_scale * m) * a_px;", "fabs(offset_scale) * a_px;"),
    "bwd_bound_offset_axis_factor_dropped": ("a_px += fabs(go[c] * ty * f);", "a_px += fabs(go[c] * f);"),
    "bwd_bound_offset_y_doubled": ("fabs(offset_scale * m) * a_py;", "2.0 * fabs(offset_scale * m) * a_py;"),
    "sm_missing_normalisation": ("for (int k = 0; k < P; ++k) o[k] = exp(m[k] - mx) / sum;",
                                 "for (int k = 0; k < P; ++k) o[k] = exp(m[k] - mx);"),
    "sm_no_max_shift": ("for (int k = 0; k < P; ++k) sum += exp(m[k] - mx);\n            for (int k = 0; k < P; ++k) o[k] = exp(m[k] - mx) / sum;",
                        "for (int k = 0; k < P; ++k) sum += exp(m[k]);\n            for (int k = 0; k < P; ++k) o[k] = exp(m[k]) / sum;"),
    "sm_first_group_only": ("const double* m = mask + r * stride + (int64_t)g * P;",
                            "const double* m = mask + r * stride;"),
    "f64_skips_center_always": ("if (s.remove_center && i == K / 2 && j == K / 2) continue;\n                const double dx",
                                "if (i == K / 2 && j == K / 2) continue;\n                const double dx"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(before) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(before, after, 1)
    csrc = tmp_path / "mut.c"
    csrc.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-shared", "-fPIC",
                    "-o", str(so), str(csrc), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, DCNV4_ORACLE_LIB=str(so))
    pins = ("test_oracle_backward.py" if name.startswith("bwd_") else
            "test_oracle_softmax.py" if name.startswith("sm_") else "test_oracle_pins.py")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-W", "ignore::RuntimeWarning",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch '{name}':\n{r.stdout[-2000:]}"
