"""The per-direction input projections of SS2D, in numpy float64.
TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it.

[SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §3.2 (parameter projection
before the selective scan), in the page's order:
  1. xs = cross_scan(x): the four scan sequences (B, 4, D, L) of §3.1;
  2. x_dbl[b,k,c,l] = sum_d xs[b,k,d,l] * x_proj_weight[k,c,d], one weight
     matrix (R + 2N, D) per direction;
  3. x_dbl is split along c into dts (R rows), Bs (N rows) and Cs (N rows),
     in that order;
  4. dt[b,k,d,l] = sum_r dts[b,k,r,l] * dt_projs_weight[k,d,r], a rank-R
     map per direction; dt_projs_bias is not added here: the selective scan
     adds it as its delta bias before the softplus;
  5. the selective scan and the merge of §3.2-§3.3 then run on
     (xs, dt, Bs, Cs) with A = -exp(A_logs), Ds and that bias.
The rank R is whatever the weight shapes say; the page sizes it as
ceil(d_model / 16) (§1, dt_rank "auto").
"""
from __future__ import annotations

import numpy as np

from .ops_numpy import cross_scan


def x_proj(x, x_proj_weight) -> np.ndarray:
    """Step 2: x (B, D, H, W), x_proj_weight (4, C, D) -> x_dbl (B, 4, C, L), scan order."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(x_proj_weight, dtype=np.float64)
    assert w.ndim == 3 and w.shape[0] == 4 and w.shape[2] == x.shape[1], (w.shape, x.shape)
    xs = cross_scan(x)
    return np.einsum("bkdl,kcd->bkcl", xs, w, optimize=True)


def project(x, x_proj_weight, dt_projs_weight, N: int):
    """Steps 1-4: returns (dt (B,4,D,L), Bs (B,4,N,L), Cs (B,4,N,L)) in float64, scan order."""
    wdt = np.asarray(dt_projs_weight, dtype=np.float64)
    x_dbl = x_proj(x, x_proj_weight)
    C = x_dbl.shape[2]
    R = C - 2 * N
    D = np.asarray(x).shape[1]
    assert R >= 1 and wdt.shape == (4, D, R), (wdt.shape, C, N)
    dts, Bs, Cs = np.split(x_dbl, [R, R + N], axis=2)
    dt = np.einsum("bkrl,kdr->bkdl", dts, wdt, optimize=True)
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
