"""The two-direction (bidirectional) selective scan, in numpy float64.
TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it.

[VSSD] page "项目概述：当视觉Transformer遇到状态空间模型" §2.2: besides the usual causal
path over the token sequence, a second path runs the same kind of recursion in
the opposite direction, obtained by changing the direction of the recursion
rather than by reversing the input.  The page fuses the two paths with a
learned gate; this path sums them, as the SS2D merge sums its directions
([SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §3.3).

Definition, for batch b, path j (0: tokens 0..L-1, 1: tokens L-1..0), channel
d (flattened c = j*D + d) and state n, with t_j(l) the token path j visits at
its step l:
    u_l      = x[b, d, t_j(l)]
    delta_l  = softplus(dt[b, j, d, l] + dt_bias[c])     (dt in the path's own step order)
    h_l      = exp(delta_l * A) * h_{l-1} + delta_l * Bs[b, j, n, l] * u_l,  h_{-1} = 0,
               A = -exp(A_log[c, n])
    out_j[l] = sum_n Cs[b, j, n, l] * h_l + Ds[c] * u_l
    y[b, d, t] = sum_j out_j[step of path j that visits t]
Both paths carry their own dt, A_log, dt_bias, Bs, Cs and Ds slices, like the
directions of SS2D.  The time loop is sequential in l, vectorised over (b, d, n).
"""
from __future__ import annotations

import numpy as np


def _softplus(v):
    return np.logaddexp(0.0, v)


def visited_token(j: int, l: int, L: int) -> int:
    """Token that path j visits at its step l."""
    return l if j == 0 else L - 1 - l


def bidir_f64(x, dt, A_log, dt_bias, Bs, Cs, Ds, want_paths: bool = False):
    """x (B, D, L); dt (B, 2, D, L); A_log (2D, N); dt_bias, Ds (2D,); Bs, Cs (B, 2, N, L).
    Returns y (B, D, L) float64, or (y, out) with out (B, 2, D, L) in each path's step order."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    x, dt, A_log, dt_bias, Bs, Cs, Ds = (f(v) for v in (x, dt, A_log, dt_bias, Bs, Cs, Ds))
    B, D, L = x.shape
    N = A_log.shape[1]
    assert dt.shape == (B, 2, D, L) and Bs.shape == (B, 2, N, L) and Cs.shape == (B, 2, N, L)
    assert A_log.shape == (2 * D, N) and dt_bias.shape == (2 * D,) and Ds.shape == (2 * D,)
    y = np.zeros((B, D, L))
    out = np.empty((B, 2, D, L))
    for j in range(2):
        A = -np.exp(A_log[j * D:(j + 1) * D])           # (D, N)
        bias = dt_bias[j * D:(j + 1) * D]
        skip = Ds[j * D:(j + 1) * D]
        h = np.zeros((B, D, N))
        for l in range(L):
            t = visited_token(j, l, L)
            u = x[:, :, t]                              # (B, D)
            delta = _softplus(dt[:, j, :, l] + bias[None, :])
            h = np.exp(delta[:, :, None] * A[None]) * h + (delta * u)[:, :, None] * Bs[:, j, None, :, l]
            o = np.sum(h * Cs[:, j, None, :, l], axis=2) + skip[None, :] * u
            out[:, j, :, l] = o
            y[:, :, t] += o
    return (y, out) if want_paths else y


def bidir_brute(x, dt, A_log, dt_bias, Bs, Cs, Ds):
    """O(L^2) unrolled form with no recurrence, for tiny inputs: out_j[l] =
    Ds u_l + sum_{i <= l} sum_n Cs[l] exp(A sum_{m=i+1..l} delta_m) delta_i Bs[i] u_i."""
    x = np.asarray(x, np.float64)
    B, D, L = x.shape
    N = np.asarray(A_log).shape[1]
    y = np.zeros((B, D, L))
    for b in range(B):
        for j in range(2):
            for d in range(D):
                c = j * D + d
                u = [float(x[b, d, visited_token(j, l, L)]) for l in range(L)]
                delta = [float(_softplus(float(dt[b, j, d, l]) + float(dt_bias[c]))) for l in range(L)]
                A = [-np.exp(float(A_log[c, n])) for n in range(N)]
                for l in range(L):
                    acc = float(Ds[c]) * u[l]
                    for i in range(l + 1):
                        s = sum(delta[i + 1:l + 1])
                        for n in range(N):
                            acc += float(Cs[b, j, n, l]) * np.exp(A[n] * s) * delta[i] * float(Bs[b, j, n, i]) * u[i]
                    y[b, d, visited_token(j, l, L)] += acc
    return y


def _paths(v):
    """(B, D, L) -> (B, 2, D, L): the tokens in each path's step order."""
    return np.stack([v, v[:, :, ::-1]], axis=1)


def bidir_backward_f64(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy):
    """Gradients of sum(dy * y) for the two-path scan above, by the chain rule along
    each path (the same derivation as the four-direction backward, with the two
    token orders as the walks):
        u_l, g_l         x and dy at the token the path visits at step l
        q_l            = Cs[n,l] g_l + a_{l+1} q_{l+1},  q_L = 0  (the state adjoint)
        dCs[n,l]       = sum_d h_l g_l,        dBs[n,l] = sum_d q_l delta_l u_l
        du_l           = sum_n q_l delta_l Bs[n,l] + Ds[c] g_l,  dx[t] = du of both paths at t
        ddt_l          = sigmoid(dt_l + dt_bias[c]) sum_n q_l (A a_l h_{l-1} + Bs[n,l] u_l)
        dA_log[c,n]    = A sum_{b,l} q_l delta_l a_l h_{l-1}
        ddt_bias[c]    = sum_{b,l} ddt_l,      dDs[c] = sum_{b,l} g_l u_l.
    Shapes as for bidir_f64, dy (B, D, L).  Returns a dict with dx, ddt, dA_log,
    ddt_bias, dBs, dCs, dDs in float64."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    x, dt, A_log, dt_bias, Bs, Cs, Ds, dy = (f(v) for v in (x, dt, A_log, dt_bias, Bs, Cs, Ds, dy))
    B, D, L = x.shape
    N = A_log.shape[1]
    u, g = _paths(x), _paths(dy)                          # (B, 2, D, L)
    pre = dt + dt_bias.reshape(2, D)[None, :, :, None]
    delta = _softplus(pre)
    A = -np.exp(A_log).reshape(2, D, N)
    a = np.exp(delta[:, :, :, None, :] * A[None, :, :, :, None])   # (B, 2, D, N, L)
    Bn, Cn = Bs[:, :, None], Cs[:, :, None]               # (B, 2, 1, N, L)
    inp = (delta * u)[:, :, :, None, :] * Bn
    h = np.empty_like(a)
    state = np.zeros(a.shape[:-1])
    for l in range(L):
        state = a[..., l] * state + inp[..., l]
        h[..., l] = state
    h_before = np.zeros_like(h)
    h_before[..., 1:] = h[..., :-1]
    q = np.empty_like(a)
    adj = np.zeros(a.shape[:-1])
    for l in range(L - 1, -1, -1):
        decay_next = a[..., l + 1] if l + 1 < L else 0.0
        adj = Cn[..., l] * g[:, :, :, None, l] + decay_next * adj
        q[..., l] = adj
    du = (q * delta[:, :, :, None, :] * Bn).sum(axis=3) + Ds.reshape(2, D)[None, :, :, None] * g
    ddt = (q * (A[None, :, :, :, None] * a * h_before + Bn * u[:, :, :, None, :])).sum(axis=3) / (1.0 + np.exp(-pre))
    dA = (q * delta[:, :, :, None, :] * a * h_before).sum(axis=(0, 4))
    dx = du[:, 0] + du[:, 1, :, ::-1]
    return {
        "dx": dx,
        "ddt": ddt,
        "dA_log": (dA * A).reshape(2 * D, N),
        "ddt_bias": ddt.sum(axis=(0, 3)).reshape(2 * D),
        "dBs": (q * (delta * u)[:, :, :, None, :]).sum(axis=2),
        "dCs": (h * g[:, :, :, None, :]).sum(axis=2),
        "dDs": (g * u).sum(axis=(0, 3)).reshape(2 * D),
    }
