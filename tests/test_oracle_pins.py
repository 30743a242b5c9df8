"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle under test is `oracle.ss2d_f64`
(plain C, fp64); `oracle.ops_numpy` and `oracle.brute` are independent
formulations used as second opinions.  Pages: [SS2D] "深入解析VMamba中的SS2D模块
从理论到代码实现" (§3.1 scan, §3.2 selective scan call, §3.3 merge, §4 direction
table, §5 test), [VSSD blog] (§3.1 convolution-kernel form), [DAMamba] (§2.1
discrete SSM, §3.1 zero initial state).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute, ops_numpy
import ss2d_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _steps(k, H, W):
    """step[h, w] = scan step at which direction k visits pixel (h, w), from the walk lists."""
    st = np.empty((H, W), dtype=np.int64)
    for l, (h, w) in enumerate(brute.walk(k, H, W)):
        st[h, w] = l
    return st


def _rand(B, D, H, W, N, seed, a_log="random"):
    return ss2d_inputs.tiny_random(B, D, H, W, N, seed, a_log=a_log)


def _run(inp, **kw):
    return oracle.ss2d_inputs_f64(inp, **kw)


def _softplus_inv(y):
    return y + math.log(-math.expm1(-y))


# ---------------------------------------------------------------- P4: hand example
@pytest.mark.parametrize("ds", [0.0, 1.0])
def test_hand_example_n1(ds):
    g = json.load(open(os.path.join(GOLDEN, "hand_n1.json")))
    x = np.array([1.0, 2.0]).reshape(1, 1, 1, 2)
    dt = np.zeros((1, 4, 1, 2))
    bias = np.full(4, math.log(math.e - 1.0))
    A_log = np.zeros((4, 1))
    Bs = np.ones((1, 4, 1, 2))
    Cs = np.ones((1, 4, 1, 2))
    Ds = np.full(4, ds)
    want = np.array(g["expected"]["Ds=%d" % int(ds)]["value"])
    for impl in (oracle.ss2d_f64, ops_numpy.ss2d, brute.ss2d):
        y = impl(x, dt, A_log, bias, Bs, Cs, Ds)
        np.testing.assert_allclose(y.reshape(-1), want, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- P1, P2
def test_bs_zero_gives_sum_of_skips_times_x():
    inp = _rand(2, 3, 4, 5, 4, seed=1)
    inp["Bs"][:] = 0.0
    inp["Ds"] = np.random.default_rng(7).uniform(0.5, 2.0, size=inp["Ds"].shape).astype(np.float32)
    y = _run(inp)
    D = inp["x"].shape[1]
    scale = inp["Ds"].astype(np.float64).reshape(4, D).sum(0)
    np.testing.assert_allclose(y, scale[None, :, None, None] * inp["x"], rtol=1e-14, atol=0)


def test_ds_and_cs_zero_give_zero():
    inp = _rand(1, 2, 3, 4, 5, seed=2)
    inp["Cs"][:] = 0.0
    inp["Ds"][:] = 0.0
    assert np.all(_run(inp) == 0.0)


# ---------------------------------------------------------------- P3: LTI closed forms
def _lti_inputs(B, D, H, W, N, seed):
    """delta, B and C constant along the sequence (per direction, channel, state)."""
    rng = np.random.default_rng(seed)
    L = H * W
    x = rng.standard_normal((B, D, H, W))
    dt = np.broadcast_to(rng.standard_normal((B, 4, D, 1)) * 0.5, (B, 4, D, L)).copy()
    bias = rng.uniform(-3, 0, 4 * D)
    A_log = rng.uniform(-1, 1.5, (4 * D, N))
    Bv = rng.standard_normal((B, 4, N, 1))
    Cv = rng.standard_normal((B, 4, N, 1))
    Bs = np.broadcast_to(Bv, (B, 4, N, L)).copy()
    Cs = np.broadcast_to(Cv, (B, 4, N, L)).copy()
    Ds = rng.standard_normal(4 * D)
    return x, dt, A_log, bias, Bs, Cs, Ds, Bv, Cv


@pytest.mark.parametrize("N", [4, 64])
def test_lti_constant_input_geometric_sum(N):
    """u constant too: h_l[n] = delta B_n u (1 - a_n^(l+1)) / (1 - a_n).  N = 64: a
    large state (the [VSSD] page's §4.1 recommends d_state 256)."""
    B, D, H, W = 2, 2, 3, 5
    x, dt, A_log, bias, Bs, Cs, Ds, Bv, Cv = _lti_inputs(B, D, H, W, N, seed=3)
    x[:] = np.random.default_rng(4).standard_normal((B, D, 1, 1))
    y = oracle.ss2d_f64(x, dt, A_log, bias, Bs, Cs, Ds)
    L = H * W
    want = np.zeros((B, D, H, W))
    l = np.arange(L)
    for b in range(B):
        for k in range(4):
            st = _steps(k, H, W)
            for d in range(D):
                c = k * D + d
                u = x[b, d, 0, 0]
                v = dt[b, k, d, 0] + bias[c]
                delta = math.log1p(math.exp(v))
                yk = np.full(L, Ds[c] * u)
                for n in range(N):
                    a = math.exp(-math.exp(A_log[c, n]) * delta)
                    yk += Cv[b, k, n, 0] * delta * Bv[b, k, n, 0] * u * (1 - a ** (l + 1)) / (1 - a)
                want[b, d] += yk[st]
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-13)


def test_lti_convolution_kernel_form():
    """[VSSD blog] §3.1: a time-invariant SSM equals a causal convolution with
    kernel K_j = sum_n C_n a_n^j (delta B_n); checked per direction on out_k."""
    B, D, H, W, N = 1, 2, 4, 3, 3
    x, dt, A_log, bias, Bs, Cs, Ds, Bv, Cv = _lti_inputs(B, D, H, W, N, seed=5)
    y, out_k = oracle.ss2d_f64(x, dt, A_log, bias, Bs, Cs, Ds, want_out_k=True)
    L = H * W
    j = np.arange(L)
    for k in range(4):
        order = brute.walk(k, H, W)
        for d in range(D):
            c = k * D + d
            u = np.array([x[0, d, h, w] for (h, w) in order])
            delta = math.log1p(math.exp(dt[0, k, d, 0] + bias[c]))
            K = np.zeros(L)
            for n in range(N):
                a = math.exp(-math.exp(A_log[c, n]) * delta)
                K += Cv[0, k, n, 0] * a ** j * delta * Bv[0, k, n, 0]
            want = np.convolve(u, K)[:L] + Ds[c] * u
            np.testing.assert_allclose(out_k[0, k, d], want, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P5: brute force
@pytest.mark.parametrize("H,W", [(2, 2), (2, 3), (3, 5), (1, 7), (7, 1)])
def test_brute_force_small_maps(H, W):
    inp = _rand(2, 2, H, W, 3, seed=10 + H * 7 + W)
    inp["Ds"] = np.random.default_rng(H * W).standard_normal(inp["Ds"].shape)
    y = _run(inp)
    yb = brute.ss2d(**inp)
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)


def test_brute_force_large_state():
    """N past 16 (blocks of states on the GPU): the O(L^2) form with N = 20."""
    inp = _rand(1, 2, 2, 3, 20, seed=77)
    inp["Ds"] = np.random.default_rng(78).standard_normal(inp["Ds"].shape)
    np.testing.assert_allclose(_run(inp), brute.ss2d(**inp), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("N,cuts", [(40, (16, 32)), (256, (16, 100, 255))])
def test_states_add_up(N, cuts):
    """y is Ds*u plus one term per state, so the forward over all N states equals the
    sum of forwards over any split of the states, the skip term taken once.  (The GPU
    runs N > 16 in blocks of 16 states and adds the blocks.)"""
    inp = _rand(2, 3, 3, 4, N, seed=N)
    inp["Ds"] = np.random.default_rng(N + 1).standard_normal(inp["Ds"].shape)
    whole = _run(inp)
    bounds = (0,) + cuts + (N,)
    parts = 0.0
    for i in range(len(bounds) - 1):
        lo, hi = bounds[i], bounds[i + 1]
        sub = dict(inp, A_log=inp["A_log"][:, lo:hi], Bs=inp["Bs"][:, :, lo:hi], Cs=inp["Cs"][:, :, lo:hi],
                   Ds=inp["Ds"] if i == 0 else np.zeros_like(inp["Ds"]))
        parts = parts + _run(sub)
    np.testing.assert_allclose(parts, whole, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("H,W,N,dtype", [(5, 3, 4, "f32"), (1, 9, 2, "f32"), (6, 6, 16, "bf16"),
                                         (4, 7, 1, "f32"), (3, 4, 48, "f32")])
def test_c_oracle_matches_tensor_op_formulation(H, W, N, dtype):
    inp = ss2d_inputs.tiny_random(2, 3, H, W, N, seed=H * 100 + W, dtype=dtype)
    y, ok = _run(inp, want_out_k=True)
    y2, ok2 = ops_numpy.ss2d(**inp, want_out_k=True)
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ok, ok2, rtol=1e-12, atol=1e-12)


def test_thread_count_does_not_change_result():
    inp = _rand(2, 5, 6, 7, 4, seed=21)
    y1 = _run(inp, nthreads=1)
    y4 = _run(inp, nthreads=4)
    assert np.array_equal(y1, y4)


# ---------------------------------------------------------------- P6, P7: symmetries
def _swap_dirs(a, perm, axis):
    return np.take(a, perm, axis=axis)


def _swap_channels(a, perm, D):
    s = a.shape
    return a.reshape((4, D) + s[1:])[perm].reshape(s)


@pytest.mark.parametrize("H,W", [(3, 5), (4, 2)])
def test_transpose_invariant(H, W):
    """Transposing the map swaps directions 0<->1 and 2<->3 and transposes y."""
    inp = _rand(2, 3, H, W, 4, seed=31 + H)
    D = inp["x"].shape[1]
    perm = [1, 0, 3, 2]
    y = _run(inp)
    t = dict(x=np.ascontiguousarray(np.swapaxes(inp["x"], 2, 3)),
             dt=_swap_dirs(inp["dt"], perm, 1), Bs=_swap_dirs(inp["Bs"], perm, 1),
             Cs=_swap_dirs(inp["Cs"], perm, 1), A_log=_swap_channels(inp["A_log"], perm, D),
             dt_bias=_swap_channels(inp["dt_bias"], perm, D), Ds=_swap_channels(inp["Ds"], perm, D))
    yt = _run(t)
    np.testing.assert_allclose(yt, np.swapaxes(y, 2, 3), rtol=1e-13, atol=1e-13)


def test_rotation_invariant():
    """Rotating the map by 180 degrees swaps directions 0<->2 and 1<->3 and rotates y."""
    inp = _rand(1, 2, 3, 4, 3, seed=41)
    D = inp["x"].shape[1]
    perm = [2, 3, 0, 1]
    y = _run(inp)
    r = dict(x=np.ascontiguousarray(inp["x"][:, :, ::-1, ::-1]),
             dt=_swap_dirs(inp["dt"], perm, 1), Bs=_swap_dirs(inp["Bs"], perm, 1),
             Cs=_swap_dirs(inp["Cs"], perm, 1), A_log=_swap_channels(inp["A_log"], perm, D),
             dt_bias=_swap_channels(inp["dt_bias"], perm, D), Ds=_swap_channels(inp["Ds"], perm, D))
    yr = _run(r)
    np.testing.assert_allclose(yr, y[:, :, ::-1, ::-1], rtol=1e-13, atol=1e-13)


def test_linear_in_x():
    inp = _rand(1, 3, 4, 4, 4, seed=51)
    x2 = np.random.default_rng(52).standard_normal(inp["x"].shape)
    y1 = _run(inp)
    y2 = _run(dict(inp, x=x2))
    y12 = _run(dict(inp, x=2.5 * inp["x"].astype(np.float64) - 0.75 * x2))
    np.testing.assert_allclose(y12, 2.5 * y1 - 0.75 * y2, rtol=1e-11, atol=1e-12)


def test_scan_and_merge_are_adjoint():
    """<CrossScan(x), o> = <x, CrossMerge(o)>: the merge is the transpose of the scan."""
    rng = np.random.default_rng(61)
    for (H, W) in [(3, 5), (6, 2), (1, 4)]:
        x = rng.standard_normal((2, 3, H, W))
        o = rng.standard_normal((2, 4, 3, H * W))
        lhs = np.sum(ops_numpy.scan_sequences(x) * o)
        rhs = np.sum(x.reshape(2, 3, H * W) * ops_numpy.merge_sequences(o, H, W))
        assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1)


def test_causality_one_hot():
    """A one-hot x at pixel p reaches out_k only at steps at or after the step that visits p."""
    H, W, D, N = 3, 4, 1, 3
    for (ph, pw) in [(0, 0), (1, 2), (2, 3)]:
        inp = _rand(1, D, H, W, N, seed=71 + ph * 4 + pw)
        inp["x"][:] = 0.0
        inp["x"][0, 0, ph, pw] = 1.0
        inp["Ds"][:] = 0.0
        _, out_k = _run(inp, want_out_k=True)
        for k in range(4):
            s = _steps(k, H, W)[ph, pw]
            assert np.all(out_k[0, k, 0, :s] == 0.0)
            assert np.all(out_k[0, k, 0, s:] != 0.0)


# ---------------------------------------------------------------- P11: the page's test
def test_page_cross_scan_assertions():
    g = json.load(open(os.path.join(GOLDEN, "page_cross_scan.json")))
    x = np.random.default_rng(81).standard_normal(g["input_shape"])
    xs = ops_numpy.scan_sequences(x)
    assert list(xs.shape) == g["output_shape"]
    for b in range(x.shape[0]):
        for c in (0, 17, 63):
            np.testing.assert_array_equal(xs[b, 0, c], x[b, c].flatten())
            np.testing.assert_array_equal(xs[b, 1, c], x[b, c].T.flatten())
            np.testing.assert_array_equal(xs[b, 2, c], x[b, c].flatten()[::-1])
            np.testing.assert_array_equal(xs[b, 3, c], x[b, c].T.flatten()[::-1])
    # the C oracle's u sequences are the same: with N states zero it returns Ds*u per direction
    inp = _rand(1, 2, 3, 5, 1, seed=82)
    inp["Bs"][:] = 0.0
    inp["Ds"][:] = 1.0
    _, out_k = _run(inp, want_out_k=True)
    np.testing.assert_array_equal(out_k[0], ops_numpy.scan_sequences(inp["x"].astype(np.float64))[0])


# ---------------------------------------------------------------- P12, P13: limits
def test_fast_decay_limit():
    """A_log = ln(1e4) and delta ~ 1 make exp(delta*A) underflow to 0: h_l = delta_l B_l u_l."""
    inp = _rand(1, 2, 3, 3, 4, seed=91)
    inp["A_log"][:] = math.log(1e4)
    inp["dt"][:] = 0.0
    inp["dt_bias"][:] = _softplus_inv(1.0)
    inp["Ds"][:] = 0.0
    _, out_k = _run(inp, want_out_k=True)
    D = 2
    delta = math.log1p(math.exp(float(inp["dt_bias"][0])))  # 1 up to the fp32 rounding of the bias
    for k in range(4):
        order = brute.walk(k, 3, 3)
        for d in range(D):
            u = np.array([inp["x"][0, d, h, w] for (h, w) in order], dtype=np.float64)
            want = (inp["Cs"][0, k].astype(np.float64) * inp["Bs"][0, k]).sum(0) * delta * u
            np.testing.assert_allclose(out_k[0, k, d], want, rtol=1e-12, atol=1e-14)


def test_single_pixel():
    """L = 1: y = sum_k (sum_n C_n delta_k B_n + D_k) u."""
    inp = _rand(2, 3, 1, 1, 5, seed=95)
    y = _run(inp)
    D = 3
    for b in range(2):
        for d in range(D):
            u = float(inp["x"][b, d, 0, 0])
            want = 0.0
            for k in range(4):
                c = k * D + d
                v = float(inp["dt"][b, k, d, 0]) + float(inp["dt_bias"][c])
                delta = math.log1p(math.exp(v))
                want += (sum(float(inp["Cs"][b, k, n, 0]) * delta * float(inp["Bs"][b, k, n, 0])
                             for n in range(5)) + float(inp["Ds"][c])) * u
            assert abs(y[b, d, 0, 0] - want) <= 1e-13 * (1 + abs(want))


def test_softplus_matches_definition():
    """delta = log(1 + e^v) over the whole range the inputs reach and beyond."""
    vs = np.concatenate([np.linspace(-40, 40, 161), [-745.0, -20.5, 0.0, 1e-9, 36.9, 700.0]])
    for v in vs:
        # L = 1, N = 1, B = C = 1, D = 0, x = 1: every direction contributes delta.
        x = np.ones((1, 1, 1, 1))
        dt = np.full((1, 4, 1, 1), v)
        y = oracle.ss2d_f64(x, dt, np.zeros((4, 1)), np.zeros(4), np.ones((1, 4, 1, 1)),
                            np.ones((1, 4, 1, 1)), np.zeros(4))
        want = 4.0 * (math.log1p(math.exp(v)) if v < 30 else v + math.log1p(math.exp(-v)))
        assert abs(y[0, 0, 0, 0] - want) <= 4e-16 * abs(want) + 1e-300, v


# ---------------------------------------------------------------- generator
def test_generator_is_deterministic_and_shaped():
    s = ss2d_inputs.CONFIGS[0]
    a = ss2d_inputs.generate(s, seed=0)
    b = ss2d_inputs.generate(s, seed=0)
    for k in a:
        assert a[k].dtype == np.float32
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (1, 16, 8, 8) and a["dt"].shape == (1, 4, 16, 64)
    assert a["Bs"].shape == (1, 4, 16, 64) and a["A_log"].shape == (64, 16)
    np.testing.assert_allclose(a["A_log"][5], np.log(np.arange(1, 17)), rtol=1e-7)
    # bias recipe: softplus(bias) lies in [1e-3, 1e-1]
    d0 = np.log1p(np.exp(a["dt_bias"].astype(np.float64)))
    assert d0.min() >= 1e-3 * (1 - 1e-5) and d0.max() <= 1e-1 * (1 + 1e-5)


def test_generator_bf16_rounding():
    s = ss2d_inputs.Shape("t", 1, 4, 3, 5, 2, "bf16")
    a = ss2d_inputs.generate(s, seed=3)
    for k in ("x", "dt", "Bs", "Cs"):
        bits = a[k].view(np.uint32)
        assert np.all((bits & 0xFFFF) == 0)
    v = np.array([1.0, 1.00390625, 1.005859375, -3.3e-5, 65504.0], np.float32)
    r = ss2d_inputs.round_to_bf16(v)
    assert r[0] == 1.0 and r[1] == 1.0  # tie rounds to even
    assert r[2] == np.float32(1.0078125)
