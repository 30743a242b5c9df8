"""Pins of the two-path (bidirectional) scan oracle, oracle/bidir.py (CPU only).

[VSSD] page "项目概述：当视觉Transformer遇到状态空间模型" §2.2 describes a forward path and
a backward path that runs the recursion in the opposite direction; the paths are
summed per token.  The oracle is pinned by a hand-worked example, an O(L^2)
unrolled form, its equality with the (separately pinned) four-direction oracle on
a one-row map whose column directions contribute nothing, the reversal
symmetry, the skip-only limit, and planted mistakes that these checks reject.
Its backward is pinned by central differences through the forward oracle and by
its equality with the (separately pinned) four-direction backward on such a map.
"""
import importlib.util
import json
import math
import os

import numpy as np
import pytest

import oracle
import ss2d_inputs
from oracle import bidir

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand(ds):
    L = 2
    x = np.array([[[1.0, 2.0]]])
    dt = np.zeros((1, 2, 1, L))
    bias = np.full(2, math.log(math.e - 1))
    A_log = np.zeros((2, 1))
    Bs = np.ones((1, 2, 1, L))
    Cs = np.ones((1, 2, 1, L))
    Ds = np.full(2, float(ds))
    return dict(x=x, dt=dt, A_log=A_log, dt_bias=bias, Bs=Bs, Cs=Cs, Ds=Ds)


@pytest.mark.parametrize("ds", [0, 1])
def test_hand_example(ds):
    g = json.load(open(os.path.join(GOLDEN, "bidir_hand.json")))
    want = np.array(g["y_ds0" if ds == 0 else "y_ds1"])
    for impl in (bidir.bidir_f64, bidir.bidir_brute):
        np.testing.assert_allclose(impl(**_hand(ds))[0, 0], want, rtol=1e-14)


@pytest.mark.parametrize("L,N", [(1, 3), (5, 2), (7, 4)])
def test_brute_force(L, N):
    inp = ss2d_inputs.bidir_random(2, 3, L, N, seed=L * 10 + N)
    np.testing.assert_allclose(bidir.bidir_f64(**inp), bidir.bidir_brute(**inp), rtol=1e-11, atol=1e-13)


def _as_cross_scan(inp):
    """The two paths as directions 0 and 2 of the four-direction forward on a 1 x L map;
    directions 1 and 3 get Cs = 0 and Ds = 0, so they add nothing."""
    x = inp["x"]
    B, D, L = x.shape
    N = inp["A_log"].shape[1]
    dt = np.zeros((B, 4, D, L))
    Bs = np.zeros((B, 4, N, L))
    Cs = np.zeros((B, 4, N, L))
    A_log = np.zeros((4 * D, N))
    bias = np.zeros(4 * D)
    Ds = np.zeros(4 * D)
    for j, k in ((0, 0), (1, 2)):
        dt[:, k] = inp["dt"][:, j]
        Bs[:, k] = inp["Bs"][:, j]
        Cs[:, k] = inp["Cs"][:, j]
        A_log[k * D:(k + 1) * D] = inp["A_log"][j * D:(j + 1) * D]
        bias[k * D:(k + 1) * D] = inp["dt_bias"][j * D:(j + 1) * D]
        Ds[k * D:(k + 1) * D] = inp["Ds"][j * D:(j + 1) * D]
    return dict(x=x.reshape(B, D, 1, L), dt=dt, A_log=A_log, dt_bias=bias, Bs=Bs, Cs=Cs, Ds=Ds)


@pytest.mark.parametrize("L,N", [(9, 5), (64, 16), (130, 33)])
def test_equals_four_direction_oracle_on_one_row(L, N):
    inp = ss2d_inputs.bidir_random(2, 4, L, N, seed=L + N)
    want = oracle.ss2d_f64(**_as_cross_scan(inp)).reshape(2, 4, L)
    np.testing.assert_allclose(bidir.bidir_f64(**inp), want, rtol=1e-12, atol=1e-13)


def test_reversal_symmetry():
    """Reversing the tokens and swapping the two paths' parameter slots reverses y."""
    inp = ss2d_inputs.bidir_random(2, 3, 11, 4, seed=7)
    D = 3
    sw = lambda a, axis: np.concatenate(np.split(a, 2, axis=axis)[::-1], axis=axis)
    rev = dict(x=inp["x"][:, :, ::-1], dt=inp["dt"][:, ::-1], Bs=inp["Bs"][:, ::-1], Cs=inp["Cs"][:, ::-1],
               A_log=sw(inp["A_log"], 0), dt_bias=sw(inp["dt_bias"], 0), Ds=sw(inp["Ds"], 0))
    assert rev["A_log"].shape == (2 * D, 4)
    np.testing.assert_allclose(bidir.bidir_f64(**rev), bidir.bidir_f64(**inp)[:, :, ::-1], rtol=1e-12,
                               atol=1e-13)


def test_bs_zero_gives_skip_only():
    inp = ss2d_inputs.bidir_random(1, 2, 6, 3, seed=3)
    inp["Bs"] = np.zeros_like(inp["Bs"])
    inp["Ds"] = np.array([0.5, -1.0, 2.0, 0.25])
    want = (inp["Ds"][:2] + inp["Ds"][2:])[None, :, None] * inp["x"].astype(np.float64)
    np.testing.assert_allclose(bidir.bidir_f64(**inp), want, rtol=1e-14)


# ---- the two-path backward (bidir_backward_f64)

def _dy(inp, seed):
    return np.random.default_rng(seed).standard_normal(np.asarray(inp["x"]).shape)


def test_backward_matches_central_differences():
    """Every gradient against central differences of sum(dy * y) through the forward
    oracle (pinned above), one input element at a time."""
    inp = {k: np.asarray(v, np.float64).copy() for k, v in ss2d_inputs.bidir_random(2, 2, 6, 3, seed=5).items()}
    dy = _dy(inp, 6)
    got = bidir.bidir_backward_f64(**inp, dy=dy)
    names = {"x": "dx", "dt": "ddt", "A_log": "dA_log", "dt_bias": "ddt_bias", "Bs": "dBs", "Cs": "dCs", "Ds": "dDs"}
    eps = 1e-6
    for name, gname in names.items():
        v = inp[name]
        num = np.zeros_like(v)
        for i in np.ndindex(v.shape):
            old = v[i]
            v[i] = old + eps
            up = np.sum(dy * bidir.bidir_f64(**inp))
            v[i] = old - eps
            down = np.sum(dy * bidir.bidir_f64(**inp))
            v[i] = old
            num[i] = (up - down) / (2 * eps)
        assert got[gname].shape == v.shape, name
        np.testing.assert_allclose(got[gname], num, rtol=1e-6, atol=1e-7 * np.max(np.abs(num)), err_msg=name)


@pytest.mark.parametrize("L,N", [(9, 5), (40, 16)])
def test_backward_equals_four_direction_backward_on_one_row(L, N):
    """The two paths as directions 0 and 2 of a 1 x L map (directions 1 and 3 add
    nothing): the (separately pinned) four-direction backward gives the same
    gradients for the two paths' slots, and dx."""
    from oracle import backward
    inp = ss2d_inputs.bidir_random(2, 3, L, N, seed=L + 2 * N)
    dy = _dy(inp, L)
    got = bidir.bidir_backward_f64(**inp, dy=dy)
    want = backward.ss2d_backward_f64(**_as_cross_scan(inp), dy=dy.reshape(2, 3, 1, L))
    D = 3
    np.testing.assert_allclose(got["dx"], want["dx"].reshape(2, D, L), rtol=1e-11, atol=1e-12)
    for j, k in ((0, 0), (1, 2)):
        np.testing.assert_allclose(got["ddt"][:, j], want["ddt"][:, k], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(got["dBs"][:, j], want["dBs"][:, k], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(got["dCs"][:, j], want["dCs"][:, k], rtol=1e-11, atol=1e-12)
        for name in ("dA_log", "ddt_bias", "dDs"):
            np.testing.assert_allclose(got[name][j * D:(j + 1) * D], want[name][k * D:(k + 1) * D], rtol=1e-11,
                                       atol=1e-12, err_msg=name)


def _pins_pass(mod) -> bool:
    try:
        for ds in (0, 1):
            g = json.load(open(os.path.join(GOLDEN, "bidir_hand.json")))
            want = np.array(g["y_ds0" if ds == 0 else "y_ds1"])
            np.testing.assert_allclose(mod.bidir_f64(**_hand(ds))[0, 0], want, rtol=1e-12)
        for L, N in ((9, 5), (64, 16)):
            inp = ss2d_inputs.bidir_random(2, 4, L, N, seed=L + N)
            want = oracle.ss2d_f64(**_as_cross_scan(inp)).reshape(2, 4, L)
            np.testing.assert_allclose(mod.bidir_f64(**inp), want, rtol=1e-10, atol=1e-12)
    except AssertionError:
        return False
    return True


SRC = bidir.__file__
MUTATIONS = {
    "backward_path_not_reversed": ("return l if j == 0 else L - 1 - l", "return l"),
    "paths_share_parameters": ("A = -np.exp(A_log[j * D:(j + 1) * D])", "A = -np.exp(A_log[0:D])"),
    "output_at_the_step_not_the_token": ("            y[:, :, t] += o", "            y[:, :, l] += o"),
    "no_skip_term": ("o = np.sum(h * Cs[:, j, None, :, l], axis=2) + skip[None, :] * u",
                     "o = np.sum(h * Cs[:, j, None, :, l], axis=2)"),
    "input_term_without_delta": ("(delta * u)[:, :, None] * Bs", "u[:, :, None] * Bs"),
}


def test_pins_pass_on_the_oracle():
    assert _pins_pass(bidir)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    path = tmp_path / "bidir_mutant.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("oracle.bidir_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    assert not _pins_pass(mod)
