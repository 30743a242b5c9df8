"""The step after the merge, in numpy float64.  TEST INFRASTRUCTURE ONLY: only
the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The HIP library never calls it and shares no code with it.

[SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §3.3: the merged y (B, D, H, W)
is transposed to channel-last (B, H, W, D).  [VSSD] §5.3 lists fusing the
LayerNorm among its deployment steps; the reading taken here is a LayerNorm
over the D channels of each pixel, with the biased variance, eps inside the
square root, and per-channel scale gamma and shift beta:
    out[b, h, w, d] = (y[b, d, h, w] - m) / sqrt(v + eps) * gamma[d] + beta[d],
    m = mean_d y[b, :, h, w],   v = mean_d (y[b, :, h, w] - m)^2.
"""
from __future__ import annotations

import numpy as np


def channel_last(y) -> np.ndarray:
    """(B, D, H, W) -> (B, H, W, D)."""
    y = np.asarray(y, dtype=np.float64)
    return np.ascontiguousarray(np.transpose(y, (0, 2, 3, 1)))


def layer_norm_channel_last(y, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """Channel-last y, normalised over its last axis (the D channels of a pixel)."""
    t = channel_last(y)
    D = t.shape[-1]
    g = np.ones(D) if gamma is None else np.asarray(gamma, dtype=np.float64)
    b = np.zeros(D) if beta is None else np.asarray(beta, dtype=np.float64)
    m = t.mean(axis=-1, keepdims=True)
    v = ((t - m) ** 2).mean(axis=-1, keepdims=True)
    return (t - m) / np.sqrt(v + eps) * g + b
