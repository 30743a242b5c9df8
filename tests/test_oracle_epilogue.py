"""Pins of the epilogue oracle (oracle/epilogue.py): a hand-worked example, the
normalisation invariants, constant pixels, the affine map per channel, a
non-square map's layout, and a planted-mistake check.
"""
import importlib.util
import json
import os

import numpy as np
import pytest

from oracle import epilogue

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pins_pass(mod) -> bool:
    try:
        fx = json.load(open(os.path.join(GOLDEN, "epilogue_hand.json")))
        y = np.array(fx["y"])
        if not np.array_equal(mod.channel_last(y), np.array(fx["transpose_only"])):
            return False
        with np.errstate(all="ignore"):
            out = mod.layer_norm_channel_last(y, fx["gamma"], fx["beta"], fx["eps"])
        if not (np.allclose(out[0, 0, 0], fx["expected"]["(0,0)"], rtol=0, atol=1e-12)
                and np.allclose(out[0, 0, 2], fx["expected"]["(0,2)"], rtol=0, atol=1e-12)):
            return False
        # a non-square map: pixel (h, w) of the output holds the channels of pixel (h, w) of y
        rng = np.random.default_rng(2)
        y = rng.standard_normal((2, 5, 3, 4))
        t = mod.channel_last(y)
        if t.shape != (2, 3, 4, 5) or any(not np.array_equal(t[1, h, w], y[1, :, h, w])
                                          for h in range(3) for w in range(4)):
            return False
        # unit scale, zero shift: every pixel has mean 0 and variance v / (v + eps)
        out = mod.layer_norm_channel_last(y, eps=1e-3)
        v = y.var(axis=1)
        return (np.allclose(out.mean(axis=-1), 0, atol=1e-12)
                and np.allclose(out.var(axis=-1), v / (v + 1e-3), rtol=1e-12))
    except (AssertionError, ValueError, IndexError):
        return False


def test_shipped_epilogue_passes_the_pins():
    assert _pins_pass(epilogue)


def test_constant_pixel_gives_the_shift():
    y = np.full((1, 4, 2, 2), 3.5)
    beta = np.array([0.1, -0.2, 0.3, 0.0])
    out = epilogue.layer_norm_channel_last(y, np.array([5.0, 6.0, 7.0, 8.0]), beta, eps=1e-5)
    assert np.allclose(out, np.broadcast_to(beta, out.shape), rtol=0, atol=0)


def test_affine_map_is_per_channel():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((1, 6, 2, 3))
    g = rng.standard_normal(6)
    b = rng.standard_normal(6)
    plain = epilogue.layer_norm_channel_last(y, eps=1e-5)
    np.testing.assert_allclose(epilogue.layer_norm_channel_last(y, g, b, eps=1e-5), plain * g + b, rtol=1e-13)


def test_shift_and_scale_invariance():
    # LayerNorm ignores a per-pixel shift and (with eps scaled) a per-pixel scale
    rng = np.random.default_rng(5)
    y = rng.standard_normal((1, 8, 3, 3))
    s = rng.uniform(0.5, 2.0, size=(1, 1, 3, 3))
    c = rng.standard_normal((1, 1, 3, 3))
    a = epilogue.layer_norm_channel_last(y, eps=0.0)
    np.testing.assert_allclose(epilogue.layer_norm_channel_last(y * s + c, eps=0.0), a, rtol=1e-10, atol=1e-12)


SRC = epilogue.__file__
MUTATIONS = {
    "statistics_over_pixels": ("m = t.mean(axis=-1, keepdims=True)", "m = t.mean(axis=(1, 2), keepdims=True)"),
    "unbiased_variance": ("v = ((t - m) ** 2).mean(axis=-1, keepdims=True)",
                          "v = ((t - m) ** 2).sum(axis=-1, keepdims=True) / (D - 1)"),
    "eps_outside_the_root": ("np.sqrt(v + eps)", "(np.sqrt(v) + eps)"),
    "scale_and_shift_swapped": ("* g + b", "* b + g"),
    "height_and_width_swapped": ("np.transpose(y, (0, 2, 3, 1))", "np.transpose(y, (0, 3, 2, 1))"),
    "no_centering": ("return (t - m) / np.sqrt", "return t / np.sqrt"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    path = tmp_path / "epilogue_mutant.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("oracle.epilogue_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    assert not _pins_pass(mod)
