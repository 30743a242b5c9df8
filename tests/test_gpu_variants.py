"""GPU parity of the forward's variants against the fp64 CPU oracles, through the C ABI:

* large state (N up to 256, run as blocks of 16 states whose outputs are summed):
  [VSSD] page "项目概述：当视觉Transformer遇到状态空间模型" §4.1 (d_state 256);
* the two-path (bidirectional) scan, ss2d_bidir_forward: [VSSD] §2.2;
* bases aligned to their element but not to 16 (fp32) / 8 (bf16) bytes, which
  take the scalar path instead of being rejected.

Tolerances as for the forward: fp32 rel-L2 <= 1e-5 and max |err| <= 1e-4 max|y|;
bf16 storage rel-L2 <= 2e-2; the scan alone (Ds = 0) 1e-4 / 5e-3.
"""
import numpy as np
import pytest

import oracle
import ss2d_inputs
from oracle import bidir as obidir

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from test_gpu_parity import check, check_scan_only, gpu_forward, slice_planes  # noqa: E402


def _lib():
    import selective_scan_crossscan_amd as ss2d
    return ss2d


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


# ------------------------------------------------------------------ N > 16
LARGE_N = [
    # B, D, H, W, N, dtype
    (1, 5, 6, 7, 17, "f32"),       # one extra state, scalar paths (L % 4 != 0)
    (2, 6, 16, 16, 32, "f32"),     # two whole blocks
    (2, 9, 28, 28, 40, "bf16"),    # a partial third block, bf16 sums kept in fp32 between blocks
    (1, 3, 33, 31, 64, "f32"),     # ragged tail
    (1, 4, 12, 16, 256, "f32"),    # d_state 256: sixteen blocks
    (1, 3, 10, 20, 256, "bf16"),
    (1, 2, 40, 64, 48, "f32"),     # transposed x (2560 steps), three blocks
    (1, 5, 72, 72, 20, "f32"),     # segmented plan, two blocks
    (2, 5, 80, 96, 33, "bf16"),    # segmented, bf16, a one-state third block
]


@pytest.mark.parametrize("B,D,H,W,N,dtype", LARGE_N)
def test_large_state(B, D, H, W, N, dtype):
    code = 1 if dtype == "bf16" else 0
    print(f"[case] large N {B}x{D}x{H}x{W} N={N} {dtype}: {_lib().describe(B, D, H, W, N, code)}", flush=True)
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=N * 7 + H, dtype=dtype)
    y = gpu_forward(inp, dtype)
    check(y, oracle.ss2d_inputs_f64(inp), dtype, f"N={N} {B}x{D}x{H}x{W}")
    inp["Ds"][:] = 0.0
    y = gpu_forward(inp, dtype)
    check_scan_only(y, oracle.ss2d_inputs_f64(inp), dtype, f"N={N} {B}x{D}x{H}x{W}")


def test_large_state_full_size_sampled():
    """VMamba-T stage-1 shape with d_state 256 (the launch configuration bench.py --n 256
    times), checked on sampled (batch, channel) planes."""
    shape = ss2d_inputs.Shape("stage1_n256", 32, 192, 56, 56, 256, "f32")
    print(f"[case] {shape}", flush=True)
    inp = ss2d_inputs.generate(shape, seed=0)
    y = gpu_forward(inp, "f32")
    bsel, dsel = [0, 31], [0, 95, 191]
    check(y[np.ix_(bsel, dsel)], oracle.ss2d_inputs_f64(slice_planes(inp, bsel, dsel)), "f32", "stage1 N=256")
    assert np.all(np.isfinite(y))


# ------------------------------------------------------------------ two-path scan
def gpu_bidir(inp, dtype):
    t = _tdt(dtype)
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(t if k in ("x", "dt", "Bs", "Cs") else torch.float32)
         .cuda() for k, v in inp.items()}
    y = _lib().bidir_forward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"])
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


BIDIR = [
    # B, D, L, N, dtype
    (1, 1, 1, 16, "f32"),
    (2, 3, 7, 5, "f32"),          # scalar paths
    (2, 17, 64, 16, "f32"),       # D past the channel block
    (1, 6, 513, 16, "f32"),
    (2, 5, 1000, 7, "bf16"),
    (4, 24, 3136, 16, "f32"),     # the stage-1 sequence length
    (1, 4, 3136, 48, "bf16"),     # three state blocks
    (1, 4, 65536, 16, "f32"),     # long: segmented (carry pass, then one launch per path)
    (1, 3, 40000, 20, "bf16"),    # segmented, bf16, two state blocks
]


@pytest.mark.parametrize("B,D,L,N,dtype", BIDIR)
def test_bidir(B, D, L, N, dtype):
    print(f"[case] bidir B={B} D={D} L={L} N={N} {dtype}: "
          f"{_lib().describe(B, D, 1, L, N, 1 if dtype == 'bf16' else 0)}", flush=True)
    inp = ss2d_inputs.bidir_random(B, D, L, N, seed=L + N, dtype=dtype)
    y = gpu_bidir(inp, dtype)
    check(y, obidir.bidir_f64(**inp), dtype, f"bidir {B}x{D}x{L} N={N}")
    inp["Ds"][:] = 0.0
    y = gpu_bidir(inp, dtype)
    check_scan_only(y, obidir.bidir_f64(**inp), dtype, f"bidir {B}x{D}x{L} N={N}")


def test_bidir_full_size_sampled():
    """The stage-1 workload as a two-path scan over its 3136 tokens (bench.py --path bidir),
    checked on batch elements 0 and 31."""
    shape = ss2d_inputs.CONFIGS[1]
    inp = ss2d_inputs.bidir_random(shape.B, shape.D, shape.L, shape.N, seed=0, a_log="s4d")
    y = gpu_bidir(inp, "f32")
    sel = [0, 31]
    sub = {k: (v[sel] if k in ("x", "dt", "Bs", "Cs") else v) for k, v in inp.items()}
    check(y[sel], obidir.bidir_f64(**sub), "f32", "bidir stage-1 sampled")


# ------------------------------------------------------------------ element-aligned bases
def _offset_tensor(arr, dtype):
    """A contiguous device tensor holding arr whose base is one element past a 256-byte
    boundary: aligned to its element, not to 16 (fp32) or 8 (bf16) bytes."""
    t = _tdt(dtype)
    flat = torch.zeros(arr.size + 64, dtype=t, device="cuda")
    view = flat[1:1 + arr.size].view(arr.shape)
    view.copy_(torch.from_numpy(np.ascontiguousarray(arr)).to(t))
    return view


OFFSET = [
    # B, D, H, W, N, dtype, which tensors sit off the vector alignment
    (2, 6, 16, 16, 16, "f32", ("x", "dt", "Bs", "Cs", "y")),
    (1, 5, 24, 32, 16, "bf16", ("x", "y")),
    (1, 3, 40, 64, 16, "f32", ("dt",)),      # would transpose x when aligned
    (1, 5, 72, 72, 16, "f32", ("Bs",)),      # would be cut into segments when aligned
    (2, 9, 28, 28, 40, "bf16", ("Cs",)),     # state blocks on the scalar path
]


@pytest.mark.parametrize("B,D,H,W,N,dtype,which", OFFSET)
def test_element_aligned_bases(B, D, H, W, N, dtype, which):
    print(f"[case] offset bases {which} {B}x{D}x{H}x{W} N={N} {dtype}", flush=True)
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=H + W + N, dtype=dtype)
    d = {}
    for k, v in inp.items():
        if k in which:
            d[k] = _offset_tensor(v, dtype)
        else:
            d[k] = torch.from_numpy(np.ascontiguousarray(v)).to(
                _tdt(dtype) if k in ("x", "dt", "Bs", "Cs") else torch.float32).cuda()
    if "y" in which:
        out = _offset_tensor(np.zeros((B, D, H, W), np.float32), dtype)
    else:
        out = torch.empty((B, D, H, W), dtype=_tdt(dtype), device="cuda")
    assert any(d[k].data_ptr() % 16 for k in which if k != "y") or out.data_ptr() % 16
    _lib().forward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"], out=out)
    torch.cuda.synchronize()
    y = out.float().cpu().numpy().astype(np.float64)
    check(y, oracle.ss2d_inputs_f64(inp), dtype, f"offset {which}")


def test_forward_from_x_with_offset_x():
    from oracle import projection
    shape = ss2d_inputs.Shape("t", 2, 32, 8, 12, 16, "f32")
    pin = ss2d_inputs.generate_projected(shape, seed=3)
    x = _offset_tensor(pin["x"], "f32")
    dev = {k: torch.from_numpy(v).cuda() for k, v in pin.items() if k != "x"}
    y = _lib().forward_from_x(x, dev["x_proj_weight"], dev["dt_projs_weight"], dev["A_log"], dev["dt_bias"],
                              dev["Ds"])
    torch.cuda.synchronize()
    check(y.double().cpu().numpy(), projection.ss2d_from_x_f64(**pin), "f32", "from_x offset x")
