"""Randomised GPU parity sweep of the module forward with a fixed seed:
shapes, channel counts (ragged and 16-byte aligned, projections of one and
several column passes), the three normalisations, remove_center, the gate
and the output projection on and off, all dtypes, offsets of 0.5 to 4
pixels' spread.  Every case is checked step by step against the module
oracle as in test_gpu_module (the operator step bit for bit)."""
import random

import pytest

from deformable_convolution_vision_dcnv4_amd import binding
from tests.test_gpu_module import check_case

pytestmark = pytest.mark.gpu


def _cases(seed, n):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        dtype = rng.choice(["f32", "f16", "bf16"])
        G = rng.choice([1, 2, 3, 4, 8])
        Cg = rng.choice([2, 4, 5, 8, 12, 16, 24, 32, 40])
        C = G * Cg
        Cin = rng.choice([3, 8, 16, 20, 24, 32, 64, 100, 160, 320])
        if dtype != "f32":
            if C % 4:
                Cg = 4 * ((Cg + 3) // 4)
                C = G * Cg
            Cin = 4 * ((Cin + 3) // 4)
        norm = rng.choice([binding.NORM_NONE, binding.NORM_GROUP, binding.NORM_LAYER])
        divs = [d for d in range(1, C + 1) if C % d == 0]
        ng = rng.choice(divs) if norm == binding.NORM_GROUP else 1
        rc, cs, op = rng.random() < 0.3, rng.random() < 0.6, rng.random() < 0.6
        Cout = rng.choice([1, 7, 16, 24, 64, 130, 200]) if op else C
        N = rng.choice([1, 2, 3])
        H, W = rng.randint(1, 24), rng.randint(1, 24)
        std = rng.choice([0.5, 1.5, 4.0])
        out.append(((N, H, W, Cin, G, Cg, Cout, norm, ng, rc, cs, op, dtype), std, 100 + len(out)))
    return out


CASES = _cases(20261204, 24)


@pytest.mark.parametrize("case,std,seed", CASES, ids=[f"case{c[2] - 100}" for c in CASES])
def test_module_sweep(case, std, seed):
    check_case(case, seed=seed, offset_std=std)
