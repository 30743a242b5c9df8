"""The SS2D forward written as the page's tensor operations, in numpy float64.
TEST INFRASTRUCTURE ONLY (second, independent oracle formulation).

[SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现":
  §3.1  cross scan: stack the plain flatten and the flatten of the H<->W
        transpose, then append both sequences flipped along L -> xs (B,4,D,L).
  §3.2  selective scan over u = xs viewed as (B, 4D, L) with delta = dts viewed
        the same way, A = -exp(A_log), per-direction B and C shared by the
        direction's D channels, D skip, delta bias added before softplus.
  §3.3  merge: flip directions 2-3 back, view directions 1 and 3 as (W, H) and
        transpose to (H, W), then sum the four.
The time loop is vectorised over (b, channel, state); it runs in order over l.
"""
from __future__ import annotations

import numpy as np


def cross_scan(x: np.ndarray) -> np.ndarray:
    """(B, D, H, W) -> (B, 4, D, L): row flatten, column flatten, and both reversed."""
    B, D, H, W = x.shape
    L = H * W
    x_hwwh = np.stack([x.reshape(B, D, L),
                       np.ascontiguousarray(np.swapaxes(x, 2, 3)).reshape(B, D, L)], axis=1)
    return np.concatenate([x_hwwh, np.flip(x_hwwh, axis=-1)], axis=1)


def cross_merge(out_y: np.ndarray, H: int, W: int) -> np.ndarray:
    """(B, 4, D, L) -> (B, D, L): undo the flips and the transpose, sum the four."""
    B, K, D, L = out_y.shape
    assert K == 4 and L == H * W
    inv_y = np.flip(out_y[:, 2:4], axis=-1)
    wh_y = np.swapaxes(out_y[:, 1].reshape(B, D, W, H), 2, 3).reshape(B, D, L)
    invwh_y = np.swapaxes(inv_y[:, 1].reshape(B, D, W, H), 2, 3).reshape(B, D, L)
    return out_y[:, 0] + inv_y[:, 0] + wh_y + invwh_y


def softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def selective_scan(u, delta, A, Bs, Cs, Ds, delta_bias):
    """u, delta (B, K*D, L); A (K*D, N); Bs, Cs (B, K, N, L); Ds, delta_bias (K*D,).
    Returns (B, K*D, L)."""
    Bsz, KD, L = u.shape
    K = Bs.shape[1]
    Dch = KD // K
    N = A.shape[1]
    delta = softplus(delta + delta_bias[None, :, None])
    # channel c = k*D + d reads the B/C of direction k
    Bc = np.repeat(Bs, Dch, axis=1)  # (B, K*D, N, L)
    Cc = np.repeat(Cs, Dch, axis=1)
    h = np.zeros((Bsz, KD, N))
    y = np.empty((Bsz, KD, L))
    for l in range(L):
        dl = delta[:, :, l]
        h = np.exp(dl[:, :, None] * A[None]) * h + (dl * u[:, :, l])[:, :, None] * Bc[:, :, :, l]
        y[:, :, l] = np.einsum("bcn,bcn->bc", h, Cc[:, :, :, l])
    return y + Ds[None, :, None] * u


def ss2d(x, dt, A_log, dt_bias, Bs, Cs, Ds, want_out_k: bool = False):
    """Whole forward in float64 via the tensor-op formulation.  x (B,D,H,W) -> (B,D,H,W)."""
    x = np.asarray(x, dtype=np.float64)
    B, D, H, W = x.shape
    L = H * W
    xs = cross_scan(x)
    out = selective_scan(xs.reshape(B, 4 * D, L), np.asarray(dt, np.float64).reshape(B, 4 * D, L),
                         -np.exp(np.asarray(A_log, np.float64)), np.asarray(Bs, np.float64),
                         np.asarray(Cs, np.float64), np.asarray(Ds, np.float64),
                         np.asarray(dt_bias, np.float64))
    out_y = out.reshape(B, 4, D, L)
    y = cross_merge(out_y, H, W).reshape(B, D, H, W)
    return (y, out_y) if want_out_k else y
