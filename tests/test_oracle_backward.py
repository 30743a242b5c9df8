"""Pins of the backward oracle (oracle/backward.py) against facts that do not
come from it: torch autograd (float64, CPU) through a forward written here from
the page's steps, central finite differences of the C oracle's forward, the
exact adjoint identity for dx (y is linear in x), and the closed form of dDs.
A mutation test plants plausible mistakes in a private copy of the module.
"""
import importlib.util

import numpy as np
import pytest

import oracle
from oracle import backward
import ss2d_inputs

torch = pytest.importorskip("torch")

GRADS = ("dx", "ddt", "dA_log", "ddt_bias", "dBs", "dCs", "dDs")


def _case(B=2, D=2, H=2, W=3, N=3, seed=0):
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=seed)
    inp = {k: v.astype(np.float64) for k, v in inp.items()}
    rng = np.random.default_rng(seed + 100)
    inp["Ds"] = rng.standard_normal(4 * D)
    inp["dt_bias"] = rng.standard_normal(4 * D) * 0.5
    dy = rng.standard_normal((B, D, H, W))
    return inp, dy


def _torch_forward(x, dt, A_log, dt_bias, Bs, Cs, Ds):
    """The forward from the page's steps in torch ops: cross scan (flatten, flatten
    of the transpose, both flipped), the recurrence per channel and state, then
    the merge (flip back, transpose back, sum)."""
    B, D, H, W = x.shape
    L = H * W
    N = A_log.shape[1]
    row = x.reshape(B, D, L)
    col = x.transpose(2, 3).reshape(B, D, L)
    xs = torch.stack([row, col, row.flip(-1), col.flip(-1)], dim=1)        # (B, 4, D, L)
    delta = torch.nn.functional.softplus(dt + dt_bias.reshape(1, 4, D, 1))
    A = -torch.exp(A_log).reshape(4, D, N)
    h = torch.zeros(B, 4, D, N, dtype=x.dtype)
    outs = []
    for l in range(L):
        dl = delta[..., l]
        h = torch.exp(dl[..., None] * A) * h + (dl * xs[..., l])[..., None] * Bs[:, :, None, :, l]
        outs.append((h * Cs[:, :, None, :, l]).sum(-1))
    ys = torch.stack(outs, dim=-1) + Ds.reshape(1, 4, D, 1) * xs
    y0, y1, y2, y3 = ys[:, 0], ys[:, 1], ys[:, 2].flip(-1), ys[:, 3].flip(-1)
    back = lambda t: t.reshape(B, D, W, H).transpose(2, 3).reshape(B, D, L)
    return (y0 + y2 + back(y1) + back(y3)).reshape(B, D, H, W)


def _autograd(inp, dy):
    names = ("x", "dt", "A_log", "dt_bias", "Bs", "Cs", "Ds")
    ts = {k: torch.tensor(inp[k], dtype=torch.float64, requires_grad=True) for k in names}
    y = _torch_forward(*(ts[k] for k in names))
    (y * torch.tensor(dy)).sum().backward()
    return {"d" + k: ts[k].grad.numpy() for k in names}


def _pins_pass(mod) -> bool:
    try:
        for shape in ((2, 2, 2, 3, 3), (1, 3, 3, 2, 2)):
            inp, dy = _case(*shape, seed=sum(shape))
            got = mod.ss2d_backward_f64(**inp, dy=dy)
            want = _autograd(inp, dy)
            for k in GRADS:
                if got[k].shape != want[k].shape or not np.allclose(got[k], want[k], rtol=1e-9, atol=1e-11):
                    return False
        # y is linear in x: <dy, y(x)> = <dx, x>
        inp, dy = _case(1, 3, 3, 4, 2, seed=9)
        y = oracle.ss2d_f64(**inp)
        dx = mod.ss2d_backward_f64(**inp, dy=dy)["dx"]
        return bool(np.isclose(np.sum(dy * y), np.sum(dx * inp["x"]), rtol=1e-12))
    except (AssertionError, ValueError, IndexError, KeyError):
        return False


def test_shipped_backward_passes_the_pins():
    assert _pins_pass(backward)


@pytest.mark.parametrize("name", ["x", "dt", "A_log", "dt_bias", "Bs", "Cs", "Ds"])
def test_central_differences_of_the_c_forward(name):
    inp, dy = _case(1, 2, 3, 2, 2, seed=21)
    grads = backward.ss2d_backward_f64(**inp, dy=dy)
    rng = np.random.default_rng(5)
    a = inp[name]
    for _ in range(4):
        idx = tuple(rng.integers(0, s) for s in a.shape)
        eps = 1e-6
        plus = {k: v.copy() for k, v in inp.items()}
        minus = {k: v.copy() for k, v in inp.items()}
        plus[name][idx] += eps
        minus[name][idx] -= eps
        num = (np.sum(dy * oracle.ss2d_f64(**plus)) - np.sum(dy * oracle.ss2d_f64(**minus))) / (2 * eps)
        assert np.isclose(grads["d" + name][idx], num, rtol=1e-6, atol=1e-8), (name, idx)


def test_skip_gradient_closed_form():
    inp, dy = _case(2, 3, 2, 2, 2, seed=3)
    got = backward.ss2d_backward_f64(**inp, dy=dy)["dDs"].reshape(4, 3)
    x, D = inp["x"], 3
    # direction k pairs dy and x at the same pixels, in whatever order it walks them
    for k in range(4):
        for d in range(D):
            assert np.isclose(got[k, d], np.sum(dy[:, d] * x[:, d]), rtol=1e-12)


SRC = backward.__file__
MUTATIONS = {
    "adjoint_decay_not_shifted": ("nxt = a[..., l + 1] if l + 1 < L else 0.0", "nxt = a[..., l]"),
    "no_sigmoid": ("ddt = ddelta * _sigmoid(pre)", "ddt = ddelta"),
    "dA_log_without_chain": ('"dA_log": (dA * A).reshape(4 * D, N)', '"dA_log": dA.reshape(4 * D, N)'),
    "B_and_C_grads_swapped": ('"dBs": dBs,\n        "dCs": dCs,', '"dBs": dCs,\n        "dCs": dBs,'),
    "state_term_sign": ("(A[None, :, :, :, None] * a * h_prev + Bk", "(-A[None, :, :, :, None] * a * h_prev + Bk"),
    "skip_missing_in_du": ("+ Ds.reshape(4, D)[None, :, :, None] * g", "+ 0.0 * g"),
    "merge_adjoint_not_scanned": ("g = scan_sequences(dy)", "g = np.repeat(dy.reshape(B, 1, D, L), 4, axis=1)"),
    "h_instead_of_h_prev": ("dA = (q * delta[:, :, :, None, :] * a * h_prev)", "dA = (q * delta[:, :, :, None, :] * a * h)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    path = tmp_path / "backward_mutant.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("oracle.backward_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    with np.errstate(all="ignore"):
        assert not _pins_pass(mod)


@pytest.mark.parametrize("dims", [(2, 3, 5, 7, 4), (1, 2, 4, 4, 3)], ids=["35_steps", "16_steps"])
def test_saved_states_match_the_c_forward(dims):
    """ss2d_states_f64 against the (separately pinned) C forward: with Ds = 0 and Cs
    one-hot in state n0, direction k's output at step l is h_l of state n0, so entry
    p of the states is that output at step 8p - 1 (and entry 0 is zero)."""
    B, D, H, W, N = dims
    L = H * W
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=sum(dims))
    st = backward.ss2d_states_f64(**{k: inp[k] for k in ("x", "dt", "A_log", "dt_bias", "Bs", "Cs")})
    P = (L + 7) // 8
    assert st.shape == (B, 4, D, N, P)
    assert np.all(st[..., 0] == 0.0)
    for n0 in range(N):
        Cs = np.zeros_like(inp["Cs"])
        Cs[:, :, n0, :] = 1.0
        _, out_k = oracle.ss2d_f64(**{**inp, "Cs": Cs, "Ds": np.zeros_like(inp["Ds"])}, want_out_k=True)
        for p in range(1, P):
            np.testing.assert_allclose(st[:, :, :, n0, p], out_k[:, :, :, 8 * p - 1], rtol=1e-12, atol=1e-14)
