"""CPU oracle for the SS2D forward path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it and shares no code with it.

Three independent formulations of the scan, and the projections, live here:
  * `ss2d_f64`      -- plain C loops in double precision (ss2d_oracle.c),
                        OpenMP across (b, d) planes only.  The reference result.
  * `ops_numpy`     -- each direction as a permutation of the pixel indices
                        (the grid of pixel numbers read along that direction),
                        the sequences gathered and the outputs scattered back
                        through it, with a vectorised time loop, in float64.
  * `brute`         -- an O(L^2) unrolled sum with no recurrence at all, for tiny
                        maps, walking the map in the orders the direction table
                        describes.
  * `projection`    -- the per-direction input projections of §3.2 (x_proj,
                        the split into dts/Bs/Cs, the rank-R dt map) in numpy
                        float64, and the forward from the feature map and
                        the projection weights built on them.
  * `epilogue`      -- the channel-last transpose after the merge and a
                        LayerNorm over the channels of each pixel, in numpy
                        float64.
  * `backward`      -- the forward's gradients by the chain rule (state
                        adjoints walked from the end), in numpy float64.
Pages: [SS2D] "深入解析VMamba中的SS2D模块从理论到代码实现" §3.1-§4.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ss2d_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2 -fopenmp) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Open a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.ss2d_oracle_f64.argtypes = [dp] * 9 + [ctypes.c_int64] * 5 + [ctypes.c_int]
    lib.ss2d_oracle_f64.restype = ctypes.c_int
    lib.ss2d_oracle_threads.argtypes = []
    lib.ss2d_oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = load_library(_LIB_PATH)
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads() -> int:
    return _load().ss2d_oracle_threads()


def ss2d_f64(x, dt, A_log, dt_bias, Bs, Cs, Ds, want_out_k: bool = False, nthreads: int = 0,
             lib=None):
    """Reference SS2D forward in float64.  Inputs are widened exactly to float64.

    x (B,D,H,W), dt (B,4,D,L), A_log (4D,N), dt_bias (4D,), Bs/Cs (B,4,N,L), Ds (4D,).
    Returns y (B,D,H,W) float64, or (y, out_k) with out_k (B,4,D,L) in scan order.
    """
    lib = lib if lib is not None else _load()
    x = _f64(x)
    B, D, H, W = x.shape
    L = H * W
    N = np.asarray(A_log).shape[1]
    dt, A_log, dt_bias, Bs, Cs, Ds = (_f64(v) for v in (dt, A_log, dt_bias, Bs, Cs, Ds))
    assert dt.shape == (B, 4, D, L), dt.shape
    assert A_log.shape == (4 * D, N) and dt_bias.shape == (4 * D,) and Ds.shape == (4 * D,)
    assert Bs.shape == (B, 4, N, L) and Cs.shape == (B, 4, N, L)
    y = np.empty((B, D, H, W), dtype=np.float64)
    out_k = np.empty((B, 4, D, L), dtype=np.float64) if want_out_k else None
    rc = lib.ss2d_oracle_f64(_ptr(x), _ptr(dt), _ptr(A_log), _ptr(dt_bias), _ptr(Bs), _ptr(Cs),
                             _ptr(Ds), _ptr(y),
                             _ptr(out_k) if out_k is not None else ctypes.POINTER(ctypes.c_double)(),
                             B, D, H, W, N, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return (y, out_k) if want_out_k else y


def ss2d_inputs_f64(inp: dict, **kw):
    """Convenience: run `ss2d_f64` on a dict as produced by ss2d_inputs.generate."""
    return ss2d_f64(inp["x"], inp["dt"], inp["A_log"], inp["dt_bias"], inp["Bs"], inp["Cs"],
                    inp["Ds"], **kw)
