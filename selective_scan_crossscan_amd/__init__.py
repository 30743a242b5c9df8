"""MI355X-native SS2D forward (VMamba CrossScan -> selective scan -> CrossMerge).

Thin Python binding over the C ABI of libss2d.so (include/ss2d.h).  It only
marshals arguments: every step of the forward runs in the HIP kernels.  PyTorch
provides device memory and the stream.  There is no CPU fallback: if the
library is missing or the tensors are not on a ROCm device, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["forward", "ss2d_forward", "project", "ss2d_project", "forward_from_x", "ss2d_forward_from_x",
           "channel_last", "ss2d_channel_last", "backward", "ss2d_backward", "measure_peaks", "describe", "bidir_forward", "ss2d_bidir_forward", "bidir_backward", "ss2d_bidir_backward", "ss2d_forward_noalloc", "trim_memory", "status_string", "version", "library_path", "lib",
           "SS2D_F32", "SS2D_BF16", "SS2DError"]

SS2D_F32 = 0
SS2D_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libss2d.so")
_lock = threading.Lock()
_lib = None


class SS2DError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libss2d call failed ({code}): {message}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


class Peaks(ctypes.Structure):
    """ss2d_peaks: rates measured on the device by ss2d_measure_peaks."""
    _fields_ = [("exp_per_s", ctypes.c_double), ("fma_per_s", ctypes.c_double),
                ("update_mix_per_s", ctypes.c_double), ("hbm_read_Bps", ctypes.c_double),
                ("hbm_copy_Bps", ctypes.c_double), ("lds_read_Bps", ctypes.c_double),
                ("compute_units", ctypes.c_int), ("state_loop_per_s", ctypes.c_double)]


def lib():
    """The loaded libss2d.so (ctypes), with argument types declared."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                                  "python -m selective_scan_crossscan_amd._build")
            L = ctypes.CDLL(_LIB_PATH)
            vp, i64 = ctypes.c_void_p, ctypes.c_int64
            L.ss2d_forward.argtypes = [vp] * 8 + [i64] * 5 + [ctypes.c_int, vp]
            L.ss2d_forward.restype = ctypes.c_int
            L.ss2d_status_string.argtypes = [ctypes.c_int]
            L.ss2d_status_string.restype = ctypes.c_char_p
            L.ss2d_last_hip_error.argtypes = []
            L.ss2d_last_hip_error.restype = ctypes.c_char_p
            L.ss2d_version.argtypes = []
            L.ss2d_version.restype = ctypes.c_int
            L.ss2d_describe.argtypes = [i64] * 5 + [ctypes.c_int, ctypes.c_char_p, i64]
            L.ss2d_describe.restype = ctypes.c_int
            L.ss2d_describe_lanes.argtypes = [i64] * 5 + [ctypes.c_int, ctypes.c_int, ctypes.c_char_p, i64]
            L.ss2d_describe_lanes.restype = ctypes.c_int
            L.ss2d_forward_lanes.argtypes = [vp] * 8 + [i64] * 5 + [ctypes.c_int, ctypes.c_int, vp]
            L.ss2d_forward_lanes.restype = ctypes.c_int
            L.ss2d_bidir_forward.argtypes = [vp] * 8 + [i64] * 4 + [ctypes.c_int, vp]
            L.ss2d_bidir_forward.restype = ctypes.c_int
            L.ss2d_forward_noalloc.argtypes = [vp] * 8 + [i64] * 5 + [ctypes.c_int, vp]
            L.ss2d_forward_noalloc.restype = ctypes.c_int
            L.ss2d_trim_memory.argtypes = []
            L.ss2d_trim_memory.restype = ctypes.c_int
            L.ss2d_project.argtypes = [vp] * 6 + [i64] * 6 + [ctypes.c_int, vp]
            L.ss2d_project.restype = ctypes.c_int
            L.ss2d_forward_from_x.argtypes = [vp] * 7 + [i64] * 6 + [ctypes.c_int, vp]
            L.ss2d_forward_from_x.restype = ctypes.c_int
            L.ss2d_channel_last.argtypes = [vp, vp, vp, ctypes.c_float, ctypes.c_int, vp] + [i64] * 4 + [
                ctypes.c_int, vp]
            L.ss2d_channel_last.restype = ctypes.c_int
            L.ss2d_backward.argtypes = [vp] * 15 + [i64] * 5 + [ctypes.c_int, vp]
            L.ss2d_backward.restype = ctypes.c_int
            L.ss2d_bidir_backward.argtypes = [vp] * 15 + [i64] * 4 + [ctypes.c_int, vp]
            L.ss2d_bidir_backward.restype = ctypes.c_int
            L.ss2d_measure_peaks.argtypes = [ctypes.POINTER(Peaks), i64, vp]
            L.ss2d_measure_peaks.restype = ctypes.c_int
            _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().ss2d_status_string(int(code)).decode()


def version() -> int:
    return lib().ss2d_version()


def describe(B, D, H, W, N, dtype=SS2D_F32, lanes: int = 0) -> str:
    """The launch plan of a forward of this shape (lanes: 0 = automatic, else 16/32/64)."""
    buf = ctypes.create_string_buffer(1024)
    if lanes:
        rc = lib().ss2d_describe_lanes(B, D, H, W, N, int(dtype), int(lanes), buf, len(buf))
    else:
        rc = lib().ss2d_describe(B, D, H, W, N, int(dtype), buf, len(buf))
    if rc != 0:
        raise SS2DError(rc, status_string(rc))
    return buf.value.decode()


def trim_memory() -> None:
    """Return the freed temporaries the library's memory pools hold to the system."""
    rc = lib().ss2d_trim_memory()
    if rc != 0:
        _raise(rc)


def ss2d_forward(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, dtype, stream, lanes: int = 0) -> int:
    """Raw C-ABI call with integer device addresses; returns the status code."""
    if lanes:
        return lib().ss2d_forward_lanes(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, int(dtype),
                                        int(lanes), stream)
    return lib().ss2d_forward(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, int(dtype), stream)


def ss2d_forward_noalloc(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, dtype, stream) -> int:
    """Raw C-ABI call of the no-allocation forward; returns the status code."""
    return lib().ss2d_forward_noalloc(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, H, W, N, int(dtype), stream)


def ss2d_bidir_forward(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, L, N, dtype, stream) -> int:
    """Raw C-ABI call with integer device addresses; returns the status code."""
    return lib().ss2d_bidir_forward(x, dt, A_log, dt_bias, Bs, Cs, Ds, y, B, D, L, N, int(dtype), stream)


def ss2d_project(x, x_proj_weight, dt_projs_weight, dt, Bs, Cs, B, D, H, W, N, R, dtype, stream) -> int:
    """Raw C-ABI call with integer device addresses; returns the status code."""
    return lib().ss2d_project(x, x_proj_weight, dt_projs_weight, dt, Bs, Cs, B, D, H, W, N, R, int(dtype), stream)


def ss2d_forward_from_x(x, x_proj_weight, dt_projs_weight, A_log, dt_bias, Ds, y, B, D, H, W, N, R, dtype,
                        stream) -> int:
    """Raw C-ABI call with integer device addresses; returns the status code."""
    return lib().ss2d_forward_from_x(x, x_proj_weight, dt_projs_weight, A_log, dt_bias, Ds, y, B, D, H, W, N, R,
                                     int(dtype), stream)


def _check_tensors(x, io, params):
    import torch

    for t in io + params:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU (no CPU fallback)")
        if t.device != x.device:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    for t in io:
        if t.dtype != x.dtype:
            raise TypeError("feature map and outputs must share one dtype")
    for t in params:
        if t.dtype != torch.float32:
            raise TypeError("weights and per-channel parameters must be float32")


def _dtype_code(x) -> int:
    import torch

    if x.dtype == torch.float32:
        return SS2D_F32
    if x.dtype == torch.bfloat16:
        return SS2D_BF16
    raise TypeError(f"unsupported dtype {x.dtype}")


def _projection_shapes(x, x_proj_weight, dt_projs_weight, N):
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    B, D, H, W = x.shape
    if dt_projs_weight.dim() != 3 or dt_projs_weight.shape[0] != 4 or dt_projs_weight.shape[1] != D:
        raise ValueError("dt_projs_weight must be (4, D, R)")
    R = dt_projs_weight.shape[2]
    if tuple(x_proj_weight.shape) != (4, R + 2 * N, D):
        raise ValueError("x_proj_weight must be (4, R + 2N, D)")
    return B, D, H, W, R


def project(x, x_proj_weight, dt_projs_weight, N: int, stream=None):
    """Per-direction input projections on torch tensors (ss2d_project).

    x (B,D,H,W) float32 or bfloat16; x_proj_weight (4, R+2N, D), dt_projs_weight (4, D, R) float32.
    Returns (dt (B,4,D,L), Bs (B,4,N,L), Cs (B,4,N,L)) in x's dtype, scan order.
    """
    import torch

    code = _dtype_code(x)
    B, D, H, W, R = _projection_shapes(x, x_proj_weight, dt_projs_weight, N)
    L = H * W
    dt = torch.empty((B, 4, D, L), dtype=x.dtype, device=x.device)
    Bs = torch.empty((B, 4, N, L), dtype=x.dtype, device=x.device)
    Cs = torch.empty((B, 4, N, L), dtype=x.dtype, device=x.device)
    _check_tensors(x, (x, dt, Bs, Cs), (x_proj_weight, dt_projs_weight))
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        rc = ss2d_project(x.data_ptr(), x_proj_weight.data_ptr(), dt_projs_weight.data_ptr(), dt.data_ptr(),
                          Bs.data_ptr(), Cs.data_ptr(), B, D, H, W, N, R, code, stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return dt, Bs, Cs


def forward_from_x(x, x_proj_weight, dt_projs_weight, A_log, dt_bias, Ds, out=None, stream=None):
    """SS2D forward from the feature map and the projection weights (ss2d_forward_from_x).

    x (B,D,H,W) float32 or bfloat16; x_proj_weight (4, R+2N, D), dt_projs_weight (4, D, R),
    A_log (4D,N), dt_bias (4D,), Ds (4D,) float32.  Returns y (B,D,H,W) in x's dtype.
    """
    import torch

    code = _dtype_code(x)
    N = A_log.shape[-1]
    B, D, H, W, R = _projection_shapes(x, x_proj_weight, dt_projs_weight, N)
    if tuple(A_log.shape) != (4 * D, N) or tuple(dt_bias.shape) != (4 * D,) or tuple(Ds.shape) != (4 * D,):
        raise ValueError("A_log must be (4D,N); dt_bias and Ds (4D,)")
    if out is None:
        out = torch.empty((B, D, H, W), dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != (B, D, H, W) or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B,D,H,W) tensor of x's dtype")
    _check_tensors(x, (x, out), (x_proj_weight, dt_projs_weight, A_log, dt_bias, Ds))
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        rc = ss2d_forward_from_x(x.data_ptr(), x_proj_weight.data_ptr(), dt_projs_weight.data_ptr(),
                                 A_log.data_ptr(), dt_bias.data_ptr(), Ds.data_ptr(), out.data_ptr(),
                                 B, D, H, W, N, R, code, stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


def ss2d_channel_last(y, gamma, beta, eps, normalize, out, B, D, H, W, dtype, stream) -> int:
    """Raw C-ABI call with integer device addresses; returns the status code."""
    return lib().ss2d_channel_last(y, gamma, beta, float(eps), int(normalize), out, B, D, H, W, int(dtype), stream)


def channel_last(y, gamma=None, beta=None, eps: float = 1e-5, normalize: bool = True, out=None, stream=None):
    """y (B,D,H,W) -> (B,H,W,D), LayerNorm over D per pixel when `normalize` (ss2d_channel_last).

    gamma, beta: (D,) float32 or None (scale 1, shift 0).  Returns the channel-last tensor in y's dtype.
    """
    import torch

    code = _dtype_code(y)
    if y.dim() != 4:
        raise ValueError("y must be (B, D, H, W)")
    B, D, H, W = y.shape
    for v in (gamma, beta):
        if v is not None and tuple(v.shape) != (D,):
            raise ValueError("gamma and beta must be (D,)")
    if out is None:
        out = torch.empty((B, H, W, D), dtype=y.dtype, device=y.device)
    elif tuple(out.shape) != (B, H, W, D) or out.dtype != y.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B,H,W,D) tensor of y's dtype")
    _check_tensors(y, (y, out), tuple(v for v in (gamma, beta) if v is not None))
    if stream is None:
        stream = torch.cuda.current_stream(y.device)
    with torch.cuda.device(y.device):
        rc = ss2d_channel_last(y.data_ptr(), gamma.data_ptr() if gamma is not None else None,
                               beta.data_ptr() if beta is not None else None, eps, 1 if normalize else 0,
                               out.data_ptr(), B, D, H, W, code, stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


def ss2d_backward(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs, B, D, H, W, N,
                  dtype, stream) -> int:
    """Raw C-ABI call with integer device addresses; returns the status code."""
    return lib().ss2d_backward(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs,
                               B, D, H, W, N, int(dtype), stream)


def ss2d_bidir_backward(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs, B, D, L, N,
                        dtype, stream) -> int:
    """Raw C-ABI call with integer device addresses; returns the status code."""
    return lib().ss2d_bidir_backward(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, dx, ddt, dA_log, ddt_bias, dBs, dCs,
                                     dDs, B, D, L, N, int(dtype), stream)


def backward(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, stream=None) -> dict:
    """Gradients of the forward given dy (ss2d_backward), tensors on one ROCm device.

    x, dt, Bs, Cs, dy: float32 or bfloat16, all the same; A_log, dt_bias, Ds: float32.
    Returns dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs (shapes and dtypes of the matching inputs)."""
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    return _backward_k(4, x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, stream)


def bidir_backward(x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, stream=None) -> dict:
    """Gradients of the two-path scan given dy (ss2d_bidir_backward): x, dy (B,D,L);
    dt (B,2,D,L), Bs/Cs (B,2,N,L) in each path's order; A_log (2D,N), dt_bias, Ds (2D,).
    Returns dx, ddt, dA_log, ddt_bias, dBs, dCs, dDs (shapes and dtypes of the matching inputs)."""
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    return _backward_k(2, x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, stream)


def _backward_k(K, x, dt, A_log, dt_bias, Bs, Cs, Ds, dy, stream) -> dict:
    import torch

    code = _dtype_code(x)
    for t in (dt, Bs, Cs, dy):
        if t.dtype != x.dtype:
            raise TypeError("x, dt, Bs, Cs and dy must share one dtype")
    if K == 4:
        B, D, H, W = x.shape
    else:
        B, D, W = x.shape
        H = 1
    N = A_log.shape[-1]
    ins = (x, dt, A_log, dt_bias, Bs, Cs, Ds, dy)
    if tuple(dy.shape) != tuple(x.shape):
        raise ValueError("dy must have x's shape")
    out = {name: torch.empty_like(t) for name, t in
           (("dx", x), ("ddt", dt), ("dA_log", A_log), ("ddt_bias", dt_bias), ("dBs", Bs), ("dCs", Cs), ("dDs", Ds))}
    io = (x, dt, Bs, Cs, dy, out["dx"], out["ddt"], out["dBs"], out["dCs"])
    _check_tensors(x, io, (A_log, dt_bias, Ds, out["dA_log"], out["ddt_bias"], out["dDs"]))
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        if K == 4:
            rc = ss2d_backward(*(t.data_ptr() for t in ins), *(t.data_ptr() for t in out.values()), B, D, H, W, N,
                               code, stream.cuda_stream)
        else:
            rc = ss2d_bidir_backward(*(t.data_ptr() for t in ins), *(t.data_ptr() for t in out.values()), B, D, W,
                                     N, code, stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


def measure_peaks(hbm_bytes: int = 1 << 30, stream: int = 0) -> dict:
    """Roofline probes on the current device (ss2d_measure_peaks); rates per second."""
    p = Peaks()
    rc = lib().ss2d_measure_peaks(ctypes.byref(p), int(hbm_bytes), stream)
    if rc != 0:
        _raise(rc)
    return {name: getattr(p, name) for name, _ in Peaks._fields_}


def _raise(rc: int):
    msg = status_string(rc)
    if rc == -8:
        msg += ": " + lib().ss2d_last_hip_error().decode()
    raise SS2DError(rc, msg)


def forward(x, dt, A_log, dt_bias, Bs, Cs, Ds, out=None, stream=None, lanes: int = 0):
    """SS2D forward on torch tensors.

    x (B,D,H,W), dt (B,4,D,H*W), Bs/Cs (B,4,N,H*W): float32 or bfloat16, all the same;
    A_log (4D,N), dt_bias (4D,), Ds (4D,): float32.  All contiguous, on one ROCm device.
    N may be 1..256.  lanes: 0 (automatic) or 16/32/64 lanes per sequence chunk.
    Returns y (B,D,H,W) in x's dtype (written into `out` if given).
    """
    return _forward_k(4, x, dt, A_log, dt_bias, Bs, Cs, Ds, out, stream, lanes)


def bidir_forward(x, dt, A_log, dt_bias, Bs, Cs, Ds, out=None, stream=None):
    """Two-direction (bidirectional) selective scan on torch tensors (ss2d_bidir_forward).

    x (B,D,L), dt (B,2,D,L), Bs/Cs (B,2,N,L): float32 or bfloat16, all the same; path 1's
    dt/Bs/Cs are in its own visiting order (token L-1-l at step l).  A_log (2D,N),
    dt_bias (2D,), Ds (2D,): float32.  Returns y (B,D,L) in x's dtype.
    """
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    B, D, L = x.shape
    y = _forward_k(2, x.reshape(B, D, 1, L), dt, A_log, dt_bias, Bs, Cs, Ds,
                   None if out is None else out.view(B, D, 1, L), stream, 0)
    return y.view(B, D, L) if out is None else out


def _forward_k(K, x, dt, A_log, dt_bias, Bs, Cs, Ds, out, stream, lanes):
    import torch

    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    B, D, H, W = x.shape
    N = A_log.shape[-1]
    if x.dtype == torch.float32:
        code = SS2D_F32
    elif x.dtype == torch.bfloat16:
        code = SS2D_BF16
    else:
        raise TypeError(f"unsupported dtype {x.dtype}")
    io = (x, dt, Bs, Cs)
    params = (A_log, dt_bias, Ds)
    for t in io + params:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU (no CPU fallback)")
        if t.device != x.device:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    for t in io:
        if t.dtype != x.dtype:
            raise TypeError("x, dt, Bs, Cs must share one dtype")
    for t in params:
        if t.dtype != torch.float32:
            raise TypeError("A_log, dt_bias, Ds must be float32")
    L = H * W
    if tuple(dt.shape) != (B, K, D, L) or tuple(Bs.shape) != (B, K, N, L) or tuple(Cs.shape) != (B, K, N, L):
        raise ValueError(f"dt must be (B,{K},D,L) and Bs, Cs (B,{K},N,L)")
    if tuple(A_log.shape) != (K * D, N) or tuple(dt_bias.shape) != (K * D,) or tuple(Ds.shape) != (K * D,):
        raise ValueError(f"A_log must be ({K}D,N); dt_bias and Ds ({K}D,)")
    if out is None:
        out = torch.empty((B, D, H, W), dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != (B, D, H, W) or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B,D,H,W) tensor of x's dtype")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    ptrs = (x.data_ptr(), dt.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(), Bs.data_ptr(), Cs.data_ptr(),
            Ds.data_ptr(), out.data_ptr())
    with torch.cuda.device(x.device):
        if K == 2:
            rc = ss2d_bidir_forward(*ptrs, B, D, L, N, code, stream.cuda_stream)
        else:
            rc = ss2d_forward(*ptrs, B, D, H, W, N, code, stream.cuda_stream, lanes=lanes)
    if rc != 0:
        _raise(rc)
    return out
