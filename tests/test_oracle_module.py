"""The module oracle against library routines, closed forms and invariants
(CPU), and planted mistakes in copies of it that the pins must catch."""
import importlib.util
import os

import pytest

from oracle import module as mod
from tests import module_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "module.py")


@pytest.mark.parametrize("pin", module_pins.PINS, ids=lambda p: p.__name__)
def test_module_oracle_pin(pin):
    pin(mod)


MUTATIONS = {
    "conv1x1_transposed": ("return np.matmul(x, w.T) + b", "return np.matmul(x, w) + b"),
    "conv1x1_bias_dropped": ("return np.matmul(x, w.T) + b", "return np.matmul(x, w.T)"),
    "gn_unbiased_variance": ("var = ((v - mean) ** 2).mean(axis=(1, 3), keepdims=True)",
                             "var = ((v - mean) ** 2).sum(axis=(1, 3), keepdims=True) / (v.shape[1] * v.shape[3] - 1)"),
    "gn_stats_per_pixel": ("mean = v.mean(axis=(1, 3), keepdims=True)", "mean = v.mean(axis=(3,), keepdims=True)"),
    "gn_eps_outside": ("y = (v - mean) / np.sqrt(var + eps)", "y = (v - mean) / (np.sqrt(var) + eps)"),
    "ln_over_space": ("mean = x.mean(axis=-1, keepdims=True)\n    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)",
                      "mean = x.mean(axis=(1, 2), keepdims=True)\n    var = ((x - mean) ** 2).mean(axis=(1, 2), keepdims=True)"),
    "dw_taps_transposed": ("out += xp[:, i:i + H, j:j + W, :] * w[:, i, j]", "out += xp[:, i:i + H, j:j + W, :] * w[:, j, i]"),
    "dw_flipped": ("out += xp[:, i:i + H, j:j + W, :] * w[:, i, j]", "out += xp[:, i:i + H, j:j + W, :] * w[:, 2 - i, 2 - j]"),
    "sigmoid_sign": ("return 1.0 / (1.0 + np.exp(-t))", "return 1.0 / (1.0 + np.exp(t))"),
    "centre_gate_swapped": ("return y * (1.0 - s) + xc * s", "return y * s + xc * (1.0 - s)"),
    "centre_gate_tiled": ("s = np.repeat(sigmoid(logits), C // G, axis=-1)", "s = np.tile(sigmoid(logits), C // G)"),
    "split_weights_first": ("return rows[..., :2 * G * P], rows[..., 2 * G * P:3 * G * P]",
                            "return rows[..., G * P:3 * G * P], rows[..., :G * P]"),
    "abs_bias_signed": ("return np.matmul(np.abs(x), np.abs(w).T) + np.abs(b)", "return np.matmul(np.abs(x), np.abs(w).T) + b"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_module_planted_mistake_is_caught(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"anchor for {name}"
    path = tmp_path / "mutated_module.py"
    path.write_text(src.replace(before, after))
    spec = importlib.util.spec_from_file_location("mutated_module", path)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    caught = 0
    for pin in module_pins.PINS:
        try:
            pin(m)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught, f"no pin caught {name}"
