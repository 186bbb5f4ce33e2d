"""The five DCNv4 forward workloads, with their synthetic input recipes.

Shapes come from the FlashInternImage-T stages (stage groups 4/8/16/32 in the
classification config quoted by the usage-guide page pwwt.cn/news/2159231,
section "实战部署指南"), a high-resolution dense-prediction map and the Stable
Diffusion latent U-Net that jsqmd.com/news/933833 section 2 modifies.  All
inputs are synthetic and seeded; no dataset or trained weight is involved.
"""
import math
from dataclasses import dataclass, field


def out_dim(n, K, stride, pad, dil):
    span = n + 2 * pad - dil * (K - 1) - 1
    return span // stride + 1 if span >= 0 else 0


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    W: int
    G: int
    Cg: int
    dtypes: tuple
    x_dist: tuple = ("normal", 1.0)
    offset_dist: tuple = ("normal", 1.0)
    mask_dist: tuple = ("normal", 1.0)
    K: int = 3
    stride: int = 1
    pad: int = 1
    dil: int = 1
    offset_scale: float = 1.0
    remove_center: bool = False
    seed: int = 0
    # offsets low-pass filtered over (2r+1) x (2r+1) output pixels (0: i.i.d.)
    offset_smooth: int = 0
    note: str = field(default="", compare=False)

    @property
    def C(self):
        return self.G * self.Cg

    @property
    def P(self):
        return self.K * self.K - (1 if self.remove_center else 0)

    def out_hw(self):
        return (out_dim(self.H, self.K, self.stride, self.pad, self.dil),
                out_dim(self.W, self.K, self.stride, self.pad, self.dil))

    def units(self):
        Ho, Wo = self.out_hw()
        return self.N * Ho * Wo * self.G

    def samples(self):
        return self.units() * self.P

    def algorithmic_bytes(self, dtype):
        """x read once + offsets + weights + out written once."""
        s = 4 if dtype == "f32" else 2
        Ho, Wo = self.out_hw()
        x = self.N * self.H * self.W * self.C
        o = self.N * Ho * Wo * self.C
        return s * (x + o + self.units() * 3 * self.P)

    def backward_bytes(self, dtype):
        """Backward: x, offsets, weights and grad_out read once (I/O type);
        grad_x, grad_offset and grad_mask written once (binary32)."""
        s = 4 if dtype == "f32" else 2
        Ho, Wo = self.out_hw()
        x = self.N * self.H * self.W * self.C
        o = self.N * Ho * Wo * self.C
        rows = self.units() * 3 * self.P
        return s * (x + o + rows) + 4 * (x + rows)

    def describe(self, dtype):
        return (f"{self.name}: N={self.N} H={self.H} W={self.W} C={self.C} "
                f"(G={self.G}, Cg={self.Cg}) K={self.K} s{self.stride} p{self.pad} "
                f"d{self.dil} {dtype}")


WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 16, 4, 16, ("f32",),
                     offset_dist=("normal", 2.0), mask_dist=("normal", 1.0),
                     note="small correctness case"),
    "fiit_stage1": Workload("fiit_stage1", 64, 56, 56, 4, 16, ("f32", "f16"),
                            offset_dist=("normal", 1.5), mask_dist=("normal", 0.5),
                            note="FlashInternImage-T stage-1 shape"),
    "fiit_stage3": Workload("fiit_stage3", 64, 14, 14, 16, 16, ("f16",),
                            offset_dist=("normal", 3.0), mask_dist=("normal", 0.5),
                            note="FlashInternImage-T stage-3 shape, heavy border clipping"),
    "hires": Workload("hires", 2, 256, 256, 8, 16, ("bf16",),
                      offset_dist=("normal", 8.0), mask_dist=("uniform", -1.0, 1.0),
                      note="high-resolution dense-prediction shape"),
    "sd_latent": Workload("sd_latent", 8, 64, 64, 8, 40, ("bf16",),
                          offset_dist=("normal", 2.0),
                          mask_dist=("normal", 1.0 / math.sqrt(8.0)),
                          note="diffusion U-Net latent shape, Cg=40"),
}


# Sensitivity input, reported beside the workloads, never instead of them:
# trained offsets come from a depthwise 3x3 and a linear projection of
# spatially correlated features, so neighbouring pixels' offsets are alike,
# where the workloads' i.i.d. offsets are the harsher case.  Same shape,
# distributions and seed as fiit_stage1; offsets box-filtered over 5 x 5
# output pixels and rescaled to the same standard deviation.
SENSITIVITY = {
    "fiit_stage1_smooth": Workload("fiit_stage1_smooth", 64, 56, 56, 4, 16, ("f16",),
                                   offset_dist=("normal", 1.5), mask_dist=("normal", 0.5),
                                   offset_smooth=2,
                                   note="stage-1 shape, spatially smooth offsets (sensitivity)"),
}


def module_bytes(wl, dtype):
    """The module forward's compulsory traffic on a workload's shape (C in,
    C out, group norm, centre gate, output projection): x_in read once and
    out written once, plus the weights (matrices in the I/O type, vectors and
    depthwise taps in binary32)."""
    s = 4 if dtype == "f32" else 2
    C, P, G = wl.C, wl.P, wl.G
    R = 3 * G * P + G
    px = wl.N * wl.H * wl.W
    return 2 * px * C * s + (C * C + R * C + C * C) * s + (4 * C + 9 * C + R + C) * 4


# Every configuration the operator is measured and parity-tested on:
# (workload, I/O type).  fiit_stage1 in f16 is the headline.
CONFIGS = (("tiny", "f32"), ("fiit_stage1", "f32"), ("fiit_stage1", "f16"), ("fiit_stage3", "f16"),
           ("hires", "bf16"), ("sd_latent", "bf16"))


def oob_fractions(wl, offset_f64):
    """Reporting statistic of a workload's offsets (float64 values of the
    inputs, [N, Ho, Wo, G*2*P]): the fraction of sampling points whose
    position lies outside (-1, H) x (-1, W) (they contribute nothing), and
    the fraction with at least one of their four corners outside the image."""
    import numpy as np
    Ho, Wo = wl.out_hw()
    P, G = wl.P, wl.G
    pts = [(i, j) for i in range(wl.K) for j in range(wl.K)
           if not (wl.remove_center and i == wl.K // 2 and j == wl.K // 2)]
    ii = np.array([i for i, _ in pts], dtype=np.float64)
    jj = np.array([j for _, j in pts], dtype=np.float64)
    o = offset_f64.reshape(wl.N, Ho, Wo, G, 2, P)
    bx = (np.arange(Wo) * wl.stride - wl.pad)[None, None, :, None, None] + jj * wl.dil
    by = (np.arange(Ho) * wl.stride - wl.pad)[None, :, None, None, None] + ii * wl.dil
    px = bx + wl.offset_scale * o[..., 0, :]
    py = by + wl.offset_scale * o[..., 1, :]
    outside = ~((px > -1) & (px < wl.W) & (py > -1) & (py < wl.H))
    fx, fy = np.floor(px), np.floor(py)
    corner_out = (fx < 0) | (fx + 1 > wl.W - 1) | (fy < 0) | (fy + 1 > wl.H - 1)
    return float(outside.mean()), float((corner_out | outside).mean())
