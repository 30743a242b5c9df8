"""Seeded synthetic inputs for the SS2D forward path.

This module is shared by the oracle side (tests, CPU baseline) and the HIP side
(tests, bench, smoke).  It draws random numbers and lays them out; it holds none
of the forward path's arithmetic (no softplus, no recurrence, no scan or merge).

Shapes and layouts (c = k*D + d is the flattened channel of direction k):
  x       (B, D, H, W)    channel-first feature map
  dt      (B, 4, D, L)    per-direction step input, in that direction's scan order
  A_log   (4*D, N)        fp32
  dt_bias (4*D,)          fp32
  Bs, Cs  (B, 4, N, L)    per-direction input/output projections, scan order
  Ds      (4*D,)          fp32

Value recipe (seed s, numpy PCG64 `default_rng(s)`, draws in this order):
  x  ~ N(0, 1)
  dt ~ N(0, 0.5)          (0.5 is the standard deviation)
  U  ~ U[0, 1) per channel, dt0 = exp(U*(ln 0.1 - ln 0.001) + ln 0.001) and
       dt_bias = dt0 + ln(-expm1(-dt0)), the inverse-softplus bias initialisation
       of the page [SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §2.1
  Bs ~ N(0, 1), Cs ~ N(0, 1)
  A_log[c, n] = ln(n + 1)  ([SS2D] §2.2, S4D-real initialisation), or, with
       a_log="random", U[-1, 2.5) per element so no structure can be exploited
  Ds = 1
Each draw is made in float64 and rounded to float32.  For bf16 configurations
x, dt, Bs and Cs are further rounded to bfloat16 (round to nearest even); both
the oracle and the GPU consume the rounded values.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    B: int
    D: int
    H: int
    W: int
    N: int = 16
    dtype: str = "f32"  # "f32" or "bf16": storage type of x, dt, Bs, Cs, y

    @property
    def L(self) -> int:
        return self.H * self.W

    @property
    def updates(self) -> int:
        """State updates of one forward pass: B * 4 * D * L * N."""
        return self.B * 4 * self.D * self.L * self.N

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes the path must move: x and y once, dt, Bs, Cs, fp32 parameters."""
        s = self.elem_bytes
        return s * self.B * self.L * (6 * self.D + 8 * self.N) + 16 * self.D * (self.N + 2)


# The five workloads: tiny, VMamba-T stage-1, stage-3, stage-2 (bf16 I/O), high-res.
CONFIGS = [
    Shape("tiny", 1, 16, 8, 8, 16, "f32"),
    Shape("vmamba_t_stage1", 32, 192, 56, 56, 16, "f32"),
    Shape("vmamba_t_stage3", 32, 768, 14, 14, 16, "f32"),
    Shape("vmamba_t_stage2_bf16", 64, 384, 28, 28, 16, "bf16"),
    Shape("highres_256", 2, 192, 256, 256, 16, "f32"),
]


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32).copy()
    out[nan] = np.float32("nan")
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def generate(shape: Shape, seed: int = 0, a_log: str = "s4d", dt_min: float = 1e-3,
             dt_max: float = 1e-1, K: int = 4) -> dict:
    """Draw one input set.  Returns float32 numpy arrays (bf16-rounded where the
    shape says so) keyed x, dt, A_log, dt_bias, Bs, Cs, Ds.  K: direction slots
    of the per-direction tensors (4 for the cross scan, 2 for the two-path scan,
    whose x is then used as (B, D, H*W))."""
    B, D, H, W, N, L = shape.B, shape.D, shape.H, shape.W, shape.N, shape.L
    rng = np.random.default_rng(seed)
    x = _f32(rng.standard_normal((B, D, H, W)))
    dt = _f32(rng.standard_normal((B, K, D, L)) * 0.5)
    U = rng.random(K * D)
    dt0 = np.exp(U * (math.log(dt_max) - math.log(dt_min)) + math.log(dt_min))
    dt_bias = _f32(dt0 + np.log(-np.expm1(-dt0)))
    Bs = _f32(rng.standard_normal((B, K, N, L)))
    Cs = _f32(rng.standard_normal((B, K, N, L)))
    if a_log == "s4d":
        A_log = _f32(np.broadcast_to(np.log(np.arange(1, N + 1, dtype=np.float64)), (K * D, N)))
    elif a_log == "random":
        A_log = _f32(rng.uniform(-1.0, 2.5, size=(K * D, N)))
    else:
        raise ValueError(f"unknown a_log recipe {a_log!r}")
    Ds = np.ones(K * D, dtype=np.float32)
    if shape.dtype == "bf16":
        x, dt, Bs, Cs = (round_to_bf16(v) for v in (x, dt, Bs, Cs))
    return dict(x=x, dt=dt, A_log=np.ascontiguousarray(A_log), dt_bias=dt_bias, Bs=Bs, Cs=Cs, Ds=Ds)


def default_rank(D: int) -> int:
    """dt rank of a block with D inner channels: ceil(d_model / 16) with
    d_model = D / 2 (expansion ratio 2), the page's "auto" sizing ([SS2D] §1)."""
    return max(1, math.ceil(D / 32))


def generate_projected(shape: Shape, seed: int = 0, R: int | None = None, dt_min: float = 1e-3,
                       dt_max: float = 1e-1) -> dict:
    """Inputs of the SS2D forward from the feature map and projection weights.

    Returns float32 arrays keyed x (B,D,H,W), x_proj_weight (4, R+2N, D),
    dt_projs_weight (4, D, R), A_log (4D, N), dt_bias (4D,), Ds (4D,).
    Recipe (seed s, PCG64, draws in this order): x ~ N(0, 1); x_proj_weight
    ~ U(-1/sqrt(D), 1/sqrt(D)) (a linear layer's default initialisation);
    dt_projs_weight ~ U(-R^-1/2, R^-1/2) (the page's "random" dt init with
    dt_scale 1, [SS2D] §2.1); dt_bias by the inverse-softplus recipe of
    `generate`; A_log[c, n] = ln(n + 1); Ds = 1.  For bf16 shapes x is
    rounded to bfloat16; the weights stay float32."""
    B, D, H, W, N = shape.B, shape.D, shape.H, shape.W, shape.N
    R = default_rank(D) if R is None else R
    rng = np.random.default_rng(seed)
    x = _f32(rng.standard_normal((B, D, H, W)))
    wx = _f32(rng.uniform(-1.0, 1.0, size=(4, R + 2 * N, D)) / math.sqrt(D))
    wdt = _f32(rng.uniform(-1.0, 1.0, size=(4, D, R)) / math.sqrt(R))
    U = rng.random(4 * D)
    dt0 = np.exp(U * (math.log(dt_max) - math.log(dt_min)) + math.log(dt_min))
    dt_bias = _f32(dt0 + np.log(-np.expm1(-dt0)))
    A_log = _f32(np.broadcast_to(np.log(np.arange(1, N + 1, dtype=np.float64)), (4 * D, N)))
    Ds = np.ones(4 * D, dtype=np.float32)
    if shape.dtype == "bf16":
        x = round_to_bf16(x)
    return dict(x=x, x_proj_weight=wx, dt_projs_weight=wdt, A_log=np.ascontiguousarray(A_log), dt_bias=dt_bias,
                Ds=Ds)


def tiny_random(B: int, D: int, H: int, W: int, N: int, seed: int, dtype: str = "f32",
                a_log: str = "random", K: int = 4) -> dict:
    """Small inputs of arbitrary shape (non-square maps, ragged lengths) for tests."""
    return generate(Shape("tiny_random", B, D, H, W, N, dtype), seed=seed, a_log=a_log, K=K)


def bidir_random(B: int, D: int, L: int, N: int, seed: int, dtype: str = "f32", a_log: str = "random") -> dict:
    """Inputs of the two-path scan: x (B, D, L) and two direction slots per tensor."""
    inp = generate(Shape("bidir", B, D, 1, L, N, dtype), seed=seed, a_log=a_log, K=2)
    inp["x"] = inp["x"].reshape(B, D, L)
    return inp
