"""The SS2D forward with the walks as index tables, in numpy float64.
TEST INFRASTRUCTURE ONLY (second, independent oracle formulation).

[SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现":
  §4    direction table: direction 0 reads the map row by row, direction 1
        column by column, directions 2 and 3 read those two orders backwards.
        Here each direction is one permutation of the pixel indices, obtained
        by reading the grid of flat pixel numbers along that direction.
  §3.1  the four input sequences are x gathered through those permutations.
  §3.2  selective scan over each sequence: delta = softplus(dt + bias),
        A = -exp(A_log), the direction's B and C shared by its D channels,
        D skip, zero initial state.
  §3.3  the merge returns every output to the pixel it was computed for
        (a scatter through the same permutation) and sums the directions.
The time loop is vectorised over (b, channel, state); it runs in order over l.
"""
from __future__ import annotations

import numpy as np


def visit_orders(H: int, W: int) -> np.ndarray:
    """(4, L) int array: entry [k, l] is the flat pixel (h*W + w) direction k reads at step l."""
    grid = np.arange(H * W).reshape(H, W)        # flat pixel number at (h, w)
    along_rows = grid.reshape(-1)                # left to right, top row first
    along_cols = grid.T.reshape(-1)              # top to bottom, left column first
    return np.stack([along_rows, along_cols, along_rows[::-1], along_cols[::-1]])


def scan_sequences(x: np.ndarray) -> np.ndarray:
    """(B, D, H, W) -> (B, 4, D, L): the sequence each direction reads, in its step order."""
    B, D, H, W = x.shape
    flat = np.asarray(x).reshape(B, D, H * W)
    order = visit_orders(H, W)
    return np.stack([flat[:, :, order[k]] for k in range(4)], axis=1)


def merge_sequences(seq: np.ndarray, H: int, W: int) -> np.ndarray:
    """(B, 4, D, L) -> (B, D, L): every step's value back at its pixel, summed over directions."""
    B, K, D, L = seq.shape
    assert K == 4 and L == H * W
    order = visit_orders(H, W)
    total = np.zeros((B, D, L), dtype=np.result_type(seq.dtype, np.float64))
    for k in range(4):
        # order[k] is a permutation, so each pixel receives exactly one value per direction
        total[:, :, order[k]] += seq[:, k]
    return total


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
        y[:, :, l] = np.sum(h * Cc[:, :, :, l], axis=2)
    return y + Ds[None, :, None] * u


def ss2d(x, dt, A_log, dt_bias, Bs, Cs, Ds, want_out_k: bool = False):
    """Whole forward in float64 via the index-table formulation.  x (B,D,H,W) -> (B,D,H,W)."""
    x = np.asarray(x, dtype=np.float64)
    B, D, H, W = x.shape
    L = H * W
    u = scan_sequences(x)
    out = selective_scan(u.reshape(B, 4 * D, L), np.asarray(dt, np.float64).reshape(B, 4 * D, L),
                         -np.exp(np.asarray(A_log, np.float64)), np.asarray(Bs, np.float64),
                         np.asarray(Cs, np.float64), np.asarray(Ds, np.float64),
                         np.asarray(dt_bias, np.float64))
    out_k = out.reshape(B, 4, D, L)
    y = merge_sequences(out_k, H, W).reshape(B, D, H, W)
    return (y, out_k) if want_out_k else y
