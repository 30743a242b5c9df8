"""Pins of the projection oracle (oracle/projection.py) against facts that do not
come from it: loops over a hand-written walk of the map, the hand-written scan
order of a 2 x 3 map, the H <-> W transpose symmetry, and a rank-one input whose
projections have a closed form.  A mutation test plants plausible mistakes in a
private copy of the module and checks that these pins reject each of them.
"""
import importlib.util
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute, projection
import ss2d_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pixel(k, l, H, W):
    """(h, w) visited at step l of direction k, walked out step by step."""
    L = H * W
    if k >= 2:
        l = L - 1 - l
    if k % 2 == 0:
        return l // W, l % W
    return l % H, l // H


def _loops(x, wx, wdt, N):
    """Plain loops: project every visited pixel, split the rows, apply the rank-R map."""
    B, D, H, W = x.shape
    L = H * W
    C = wx.shape[1]
    R = C - 2 * N
    dt = np.zeros((B, 4, D, L))
    Bs = np.zeros((B, 4, N, L))
    Cs = np.zeros((B, 4, N, L))
    for b in range(B):
        for k in range(4):
            for l in range(L):
                h, w = _pixel(k, l, H, W)
                row = [sum(float(wx[k, c, d]) * float(x[b, d, h, w]) for d in range(D)) for c in range(C)]
                for n in range(N):
                    Bs[b, k, n, l] = row[R + n]
                    Cs[b, k, n, l] = row[R + N + n]
                for d in range(D):
                    dt[b, k, d, l] = sum(float(wdt[k, d, r]) * row[r] for r in range(R))
    return dt, Bs, Cs


def _case(seed=3, B=2, D=3, H=2, W=3, N=2, R=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, D, H, W))
    wx = rng.standard_normal((4, R + 2 * N, D))
    wdt = rng.standard_normal((4, D, R))
    return x, wx, wdt, N


def _pins_pass(mod) -> bool:
    try:
        # loops on a non-square map
        x, wx, wdt, N = _case()
        got = mod.project(x, wx, wdt, N)
        for g, e in zip(got, _loops(x, wx, wdt, N)):
            if g.shape != e.shape or not np.allclose(g, e, rtol=1e-12, atol=1e-12):
                return False
        # the hand-written walk of a 2 x 3 map, through identity weights
        fx = json.load(open(os.path.join(GOLDEN, "projection_walk.json")))
        H, W = fx["H"], fx["W"]
        N, R = 1, 1
        D = R + 2 * N
        xm = np.broadcast_to(np.arange(H * W, dtype=np.float64).reshape(1, 1, H, W), (1, D, H, W))
        eye = np.broadcast_to(np.eye(D), (4, D, D))
        dt, Bs, Cs = mod.project(xm, eye, np.ones((4, D, R)), N)
        want = np.array(fx["directions"], dtype=np.float64)
        if not (np.array_equal(Bs[0, :, 0], want) and np.array_equal(Cs[0, :, 0], want)
                and np.array_equal(dt[0, :, 1], want)):
            return False
        # transposing the map exchanges the row and column directions
        x, wx, wdt, N = _case(seed=4, H=3, W=2)
        perm = [1, 0, 3, 2]
        a = mod.project(x, wx, wdt, N)
        t = mod.project(np.swapaxes(x, 2, 3), wx[perm], wdt[perm], N)
        return all(np.allclose(u[:, perm], v, rtol=1e-12, atol=1e-12) for u, v in zip(a, t))
    except (AssertionError, ValueError, IndexError):
        return False


def test_shipped_projection_passes_the_pins():
    assert _pins_pass(projection)


def test_rank_one_map_has_closed_form_projections():
    # x[b,d,h,w] = u[d] * s[h,w]: every projected row is (w . u) times s along the walk
    rng = np.random.default_rng(7)
    D, H, W, N, R = 5, 3, 4, 2, 3
    u = rng.standard_normal(D)
    s = rng.standard_normal((H, W))
    x = (u[:, None, None] * s[None])[None]
    wx = rng.standard_normal((4, R + 2 * N, D))
    wdt = rng.standard_normal((4, D, R))
    dt, Bs, Cs = projection.project(x, wx, wdt, N)
    for k in range(4):
        walk = np.array([s[_pixel(k, l, H, W)] for l in range(H * W)])
        proj = wx[k] @ u
        np.testing.assert_allclose(Bs[0, k], np.outer(proj[R:R + N], walk), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(Cs[0, k], np.outer(proj[R + N:], walk), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dt[0, k], np.outer(wdt[k] @ proj[:R], walk), rtol=1e-12, atol=1e-12)


def test_forward_from_x_matches_the_brute_force_scan():
    # the composition, with the scan side checked by the O(L^2) brute force
    rng = np.random.default_rng(11)
    x, wx, wdt, N = _case(seed=12, B=1, D=2, H=2, W=3, N=2, R=2)
    A_log = rng.uniform(-1, 1.5, size=(4 * 2, N))
    bias = rng.standard_normal(4 * 2) * 0.3
    Ds = rng.standard_normal(4 * 2)
    y = projection.ss2d_from_x_f64(x, wx, wdt, A_log, bias, Ds)
    dt, Bs, Cs = _loops(x, wx, wdt, N)
    np.testing.assert_allclose(y, brute.ss2d(x, dt, A_log, bias, Bs, Cs, Ds), rtol=1e-10, atol=1e-12)


def test_abs_bound_dominates_every_output():
    x, wx, wdt, N = _case(seed=13)
    for v, bound in zip(projection.project(x, wx, wdt, N), projection.project_abs(x, wx, wdt, N)):
        assert np.all(np.abs(v) <= bound * (1 + 1e-12))


def test_generated_weights_follow_the_recipe():
    shape = ss2d_inputs.Shape("t", 2, 64, 4, 5, 16, "f32")
    inp = ss2d_inputs.generate_projected(shape, seed=1)
    R = ss2d_inputs.default_rank(64)
    assert R == 2
    assert inp["x_proj_weight"].shape == (4, R + 32, 64) and inp["dt_projs_weight"].shape == (4, 64, R)
    assert np.abs(inp["x_proj_weight"]).max() <= 1 / 8 and np.abs(inp["dt_projs_weight"]).max() <= R ** -0.5
    again = ss2d_inputs.generate_projected(shape, seed=1)
    assert all(np.array_equal(inp[k], again[k]) for k in inp)


SRC = projection.__file__
MUTATIONS = {
    "split_order_swapped": ("rows_dt, rows_B, rows_C = slice(0, R), slice(R, R + N), slice(R + N, C)",
                            "rows_dt, rows_B, rows_C = slice(2 * N, C), slice(0, N), slice(N, 2 * N)"),
    "B_and_C_swapped": ("Bs, Cs = proj[:, :, rows_B], proj[:, :, rows_C]", "Bs, Cs = proj[:, :, rows_C], proj[:, :, rows_B]"),
    "no_cross_scan": ("    seq = scan_sequences(x)", "    seq = np.repeat(x.reshape(x.shape[0], 1, x.shape[1], -1), 4, axis=1)"),
    "one_weight_for_all_directions": ("np.matmul(w[k], seq[:, k])", "np.matmul(w[0], seq[:, k])"),
    "dt_map_transposed": ("np.matmul(wdt[k], low_rank[:, k])", "np.matmul(wdt[k], low_rank[:, k, ::-1])"),
    "dt_directions_crossed": ("np.matmul(wdt[k], low_rank[:, k])", "np.matmul(wdt[k ^ 1], low_rank[:, k])"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    path = tmp_path / "projection_mutant.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("oracle.projection_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    assert not _pins_pass(mod)
