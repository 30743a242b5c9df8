"""The SS2D forward's gradients, in numpy float64.  TEST INFRASTRUCTURE ONLY:
only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The HIP library never calls it and shares no code with it.

The forward ([SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §3.1-§3.3): per
batch b, direction k, channel c = k*D + d and state n, along the scan order l,
    u_l = x at the pixel visited at l,   g_l = dy at that pixel (the merge's
    adjoint: the merge adds each direction's output at its pixel),
    delta_l = softplus(dt_l + dt_bias[c]),   A = -exp(A_log[c, n]),
    a_l = exp(delta_l * A),   h_l = a_l h_{l-1} + delta_l Bs[n,l] u_l,  h_{-1} = 0,
    out_l = sum_n Cs[n,l] h_l + Ds[c] u_l.
Its reverse-mode derivative, by the chain rule, with the state adjoint
    q_l = Cs[n,l] g_l + a_{l+1} q_{l+1},   q_L = 0   (walked from the end),
gives
    dCs[n,l]   += h_l g_l                          (summed over d)
    dBs[n,l]   += q_l delta_l u_l                  (summed over d)
    du_l        = sum_n q_l delta_l Bs[n,l] + Ds[c] g_l
    ddelta_l    = sum_n q_l (A a_l h_{l-1} + Bs[n,l] u_l)
    dA          = sum_l q_l delta_l a_l h_{l-1},   dA_log = dA * A
    dDs[c]      = sum_l g_l u_l
    ddt_l       = ddelta_l * sigmoid(dt_l + dt_bias[c]),   ddt_bias[c] = sum_l ddt_l
and dx is the merge of du: each direction's du added at the pixel it visits.
Sums over b are taken for the per-channel parameters.
"""
from __future__ import annotations

import numpy as np

from .ops_numpy import merge_sequences, scan_sequences


def _sigmoid(v):
    return 0.5 * (1.0 + np.tanh(0.5 * v))


def ss2d_backward_f64(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy):
    """Gradients of sum(dy * y) with respect to every input of the forward.

    Shapes as for the forward: x (B,D,H,W), dt (B,4,D,L), A_log (4D,N), dt_bias (4D,),
    Bs/Cs (B,4,N,L), Ds (4D,), dy (B,D,H,W).  Returns a dict with dx, ddt, dA_log,
    ddt_bias, dBs, dCs, dDs (float64, same shapes as the inputs)."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    x, dt, A_log, dt_bias, Bs, Cs, Ds, dy = (f(v) for v in (x, dt, A_log, dt_bias, Bs, Cs, Ds, dy))
    B, D, H, W = x.shape
    L = H * W
    N = A_log.shape[1]
    u = scan_sequences(x)             # (B, 4, D, L)
    g = scan_sequences(dy)            # the merge's adjoint
    bias = dt_bias.reshape(4, D)
    pre = dt + bias[None, :, :, None]
    delta = np.logaddexp(0.0, pre)    # (B, 4, D, L)
    A = -np.exp(A_log).reshape(4, D, N)
    Bk = Bs[:, :, None, :, :]         # (B, 4, 1, N, L)
    Ck = Cs[:, :, None, :, :]
    a = np.exp(delta[:, :, :, None, :] * A[None, :, :, :, None])   # (B, 4, D, N, L)
    binp = delta[:, :, :, None, :] * Bk * u[:, :, :, None, :]
    # forward states, kept for every step
    h = np.empty_like(a)
    hp = np.zeros(a.shape[:-1])
    for l in range(L):
        hp = a[..., l] * hp + binp[..., l]
        h[..., l] = hp
    h_prev = np.concatenate([np.zeros(a.shape[:-1] + (1,)), h[..., :-1]], axis=-1)
    # state adjoints, from the end
    q = np.empty_like(a)
    qn = np.zeros(a.shape[:-1])
    gk = g[:, :, :, None, :]
    for l in range(L - 1, -1, -1):
        nxt = a[..., l + 1] if l + 1 < L else 0.0
        qn = Ck[..., l] * gk[..., l] + nxt * qn
        q[..., l] = qn
    dCs = (h * gk).sum(axis=2)
    dBs = (q * delta[:, :, :, None, :] * u[:, :, :, None, :]).sum(axis=2)
    du = (q * delta[:, :, :, None, :] * Bk).sum(axis=3) + Ds.reshape(4, D)[None, :, :, None] * g
    ddelta = (q * (A[None, :, :, :, None] * a * h_prev + Bk * u[:, :, :, None, :])).sum(axis=3)
    dA = (q * delta[:, :, :, None, :] * a * h_prev).sum(axis=(0, 4))     # (4, D, N)
    ddt = ddelta * _sigmoid(pre)
    return {
        "dx": merge_sequences(du, H, W).reshape(B, D, H, W),
        "ddt": ddt,
        "dA_log": (dA * A).reshape(4 * D, N),
        "ddt_bias": ddt.sum(axis=(0, 3)).reshape(4 * D),
        "dBs": dBs,
        "dCs": dCs,
        "dDs": (g * u).sum(axis=(0, 3)).reshape(4 * D),
    }


def ss2d_states_f64(x, dt, A_log, dt_bias, Bs, Cs, every: int = 8):
    """The states h of the forward's recurrence (module docstring) entering every
    `every`-th step of each direction's walk: out[b, k, d, n, p] = h_{every*p - 1}
    (0 for p = 0), p = 0 .. ceil(L/every) - 1.  Shapes as for the forward; Cs is
    not used (the states do not depend on it) and is taken for a uniform call."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    x, dt, A_log, dt_bias, Bs = (f(v) for v in (x, dt, A_log, dt_bias, Bs))
    B, D, H, W = x.shape
    L = H * W
    N = A_log.shape[1]
    u = scan_sequences(x)                                            # (B, 4, D, L)
    delta = np.logaddexp(0.0, dt + dt_bias.reshape(4, D)[None, :, :, None])
    A = -np.exp(A_log).reshape(4, D, N)
    P = (L + every - 1) // every
    out = np.zeros((B, 4, D, N, P))
    h = np.zeros((B, 4, D, N))
    for l in range(L):
        if l % every == 0:
            out[..., l // every] = h
        a = np.exp(delta[:, :, :, None, l] * A[None])
        h = a * h + (delta[:, :, :, l] * u[:, :, :, l])[:, :, :, None] * Bs[:, :, None, :, l]
    return out
