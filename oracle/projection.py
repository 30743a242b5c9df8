"""The per-direction input projections of SS2D, in numpy float64.
TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it.

[SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §3.2 (parameter projection
before the selective scan), in the page's order:
  1. the four scan sequences (B, 4, D, L) of §3.1, read through the
     direction table's pixel orders;
  2. per direction k, its own (R + 2N) x D weight matrix applied to the D
     channels of every step's pixel;
  3. of those R + 2N projected rows, the first R are the low-rank step input,
     the next N are Bs and the last N are Cs;
  4. per direction k, its own D x R matrix maps the R low-rank rows to the
     D channels' dt; the dt bias is not added here: the selective scan adds
     it as its delta bias before the softplus;
  5. the selective scan and the merge of §3.2-§3.3 then run on
     (the sequences, dt, Bs, Cs) with A = -exp(A_log), Ds and that bias.
The rank R is whatever the weight shapes say; the page sizes it as
ceil(d_model / 16) (§1, dt_rank "auto").
"""
from __future__ import annotations

import numpy as np

from .ops_numpy import scan_sequences


def x_proj(x, x_proj_weight) -> np.ndarray:
    """Step 2: x (B, D, H, W), x_proj_weight (4, C, D) -> (B, 4, C, L) in scan order:
    entry [b, k, c, l] is row c of direction k's weight matrix applied to the D
    channels of the pixel that direction reads at step l."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(x_proj_weight, dtype=np.float64)
    assert w.ndim == 3 and w.shape[0] == 4 and w.shape[2] == x.shape[1], (w.shape, x.shape)
    seq = scan_sequences(x)                          # (B, 4, D, L)
    out = np.empty((x.shape[0], 4, w.shape[1], seq.shape[-1]))
    for k in range(4):
        out[:, k] = np.matmul(w[k], seq[:, k])       # (C, D) times (B, D, L)
    return out


def project(x, x_proj_weight, dt_projs_weight, N: int):
    """Steps 1-4: returns (dt (B,4,D,L), Bs (B,4,N,L), Cs (B,4,N,L)) in float64, scan order."""
    wdt = np.asarray(dt_projs_weight, dtype=np.float64)
    proj = x_proj(x, x_proj_weight)
    C = proj.shape[2]
    R = C - 2 * N
    D = np.asarray(x).shape[1]
    assert R >= 1 and wdt.shape == (4, D, R), (wdt.shape, C, N)
    # which projected rows are which: the low-rank step input first, then B, then C
    rows_dt, rows_B, rows_C = slice(0, R), slice(R, R + N), slice(R + N, C)
    low_rank = proj[:, :, rows_dt]                   # (B, 4, R, L)
    Bs, Cs = proj[:, :, rows_B], proj[:, :, rows_C]
    dt = np.empty((proj.shape[0], 4, D, proj.shape[-1]))
    for k in range(4):
        dt[:, k] = np.matmul(wdt[k], low_rank[:, k])  # (D, R) times (B, R, L)
    return dt, np.ascontiguousarray(Bs), np.ascontiguousarray(Cs)


def project_abs(x, x_proj_weight, dt_projs_weight, N: int):
    """The same contractions over absolute values: |dt|, |Bs|, |Cs| bounds of the form
    sum |w| |x| that scale the rounding-error bound of any evaluation order."""
    return project(np.abs(np.asarray(x, dtype=np.float64)), np.abs(np.asarray(x_proj_weight, dtype=np.float64)),
                   np.abs(np.asarray(dt_projs_weight, dtype=np.float64)), N)


def ss2d_from_x_f64(x, x_proj_weight, dt_projs_weight, A_log, dt_bias, Ds, **kw):
    """Steps 1-5: the SS2D forward from the feature map and the projection weights."""
    from . import ss2d_f64
    N = np.asarray(A_log).shape[1]
    dt, Bs, Cs = project(x, x_proj_weight, dt_projs_weight, N)
    return ss2d_f64(x, dt, A_log, dt_bias, Bs, Cs, Ds, **kw)
