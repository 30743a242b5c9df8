"""C-ABI contract of libss2d.so, checked on the CPU (no device work).

The library must load without a GPU, export every function include/ss2d.h
declares, and reject bad arguments with the documented codes before touching
the device.  Fake (never dereferenced) addresses are used for pointers.

Calls that pass validation reach the device query and report SS2D_ERR_NO_DEVICE
(-7) here; on a machine with a GPU the same calls would launch kernels on the
fake addresses, so every test that expects -7 is skipped where a device exists.
"""
import ctypes
import os
import re

import pytest

import selective_scan_crossscan_amd as ss2d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss2d.h")


def _no_device_here():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


NO_DEVICE = _no_device_here()
# valid calls launch kernels where a GPU exists: only run them where none does
needs_no_device = pytest.mark.skipif(not NO_DEVICE, reason="a valid call would launch kernels on fake addresses")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ss2d_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert names == sorted(["ss2d_forward", "ss2d_forward_lanes", "ss2d_forward_noalloc", "ss2d_bidir_forward",
                            "ss2d_status_string",
                            "ss2d_last_hip_error", "ss2d_version", "ss2d_describe", "ss2d_describe_lanes",
                            "ss2d_trim_memory", "ss2d_measure_peaks", "ss2d_project", "ss2d_forward_from_x",
                            "ss2d_channel_last", "ss2d_backward", "ss2d_bidir_backward"])
    lib = ctypes.CDLL(ss2d.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings():
    assert ss2d.version() >= 10000
    for code in range(0, -10, -1):
        s = ss2d.status_string(code)
        assert isinstance(s, str) and s
    assert ss2d.status_string(123) == "unknown status"
    assert ss2d.lib().ss2d_last_hip_error() is not None


def test_describe_plans_the_workloads():
    s = ss2d.describe(32, 192, 56, 56, 16, ss2d.SS2D_F32)
    assert "lanes_per_seq=32" in s and "chans_per_block=8" in s and "blocks=768" in s
    # the fp32 column plane, then x transposed
    assert f"scratch_bytes={2 * 32 * 192 * 3136 * 4}" in s and "x_transposed=1 plane_transposed=0" in s
    # small maps gather x in place
    s = ss2d.describe(64, 384, 28, 28, 16, ss2d.SS2D_BF16)
    assert f"scratch_bytes={2 * 64 * 384 * 784 * 4}" in s and "x_transposed=0" in s
    s = ss2d.describe(32, 768, 14, 14, 16, ss2d.SS2D_F32)
    assert "lanes_per_seq=16" in s and "chans_per_block=16" in s
    assert "segments=1 x_transposed=0 plane_transposed=0" in s
    # rows that are not 16-byte aligned keep x in place
    assert "x_transposed=0" in ss2d.describe(2, 16, 5, 7, 16, ss2d.SS2D_F32)


def test_describe_segmented_plan_includes_transposed_copies():
    """256x256 maps are cut into segments; their temporary adds the segment maps,
    a transposed x (storage type) and a transposed fp32 merge plane, 256-byte aligned."""
    B, D, L = 2, 192, 256 * 256
    s = ss2d.describe(B, D, 256, 256, 16, ss2d.SS2D_F32)
    fields = dict(kv.split("=") for kv in s.split())
    nseg = int(fields["segments"])
    assert nseg > 1 and fields["x_transposed"] == "1" and fields["plane_transposed"] == "1"
    up = lambda v: (v + 255) // 256 * 256
    base = B * D * L * 4 + B * 4 * D * nseg * 2 * 16 * 4
    xt = up(base)
    pct = up(xt + B * D * L * 4)
    assert int(fields["scratch_bytes"]) == pct + B * D * L * 4


def test_lanes_per_call():
    """The lanes choice is an argument of the call, not library state."""
    assert "lanes_per_seq=64" in ss2d.describe(32, 192, 56, 56, 16, lanes=64)
    assert "lanes_per_seq=16" in ss2d.describe(32, 192, 56, 56, 16, lanes=16)
    assert "lanes_per_seq=32" in ss2d.describe(32, 192, 56, 56, 16)   # unaffected by the calls above
    buf = ctypes.create_string_buffer(512)
    assert ss2d.lib().ss2d_describe_lanes(2, 3, 4, 5, 16, 0, 48, buf, len(buf)) == -2


def test_describe_state_blocks():
    """N > 16 runs over blocks of 16 states, in the forward and the backward alike (the
    backward's segments and channel blocks per workgroup do not depend on N)."""
    f = dict(kv.split("=") for kv in ss2d.describe(2, 32, 8, 8, 256).split())
    assert f["state_blocks"] == "16" and f["backward_segments"] == "1"
    f = dict(kv.split("=") for kv in ss2d.describe(2, 32, 8, 8, 17).split())
    assert f["state_blocks"] == "2"
    f = dict(kv.split("=") for kv in ss2d.describe(2, 32, 8, 8, 16).split())
    assert f["state_blocks"] == "1" and f["backward_segments"] == "1"


def test_describe_lanes_rule():
    # 16 lanes beyond 512 steps when the 16-channel blocks give >= 768 workgroups
    # and at most 64 steps are left after whole 256-step chunks
    assert "lanes_per_seq=16" in ss2d.describe(64, 384, 28, 28, 16, ss2d.SS2D_BF16)  # 1536 blocks, 16 left
    assert "lanes_per_seq=16" in ss2d.describe(32, 384, 40, 40, 16)   # 768 blocks, 64 left
    assert "lanes_per_seq=32" in ss2d.describe(32, 192, 28, 28, 16)   # 384 blocks
    assert "lanes_per_seq=32" in ss2d.describe(32, 768, 44, 44, 16)   # 144 left
    assert "lanes_per_seq=16" in ss2d.describe(1, 8, 15, 20, 16)      # under 512 steps
    assert "lanes_per_seq=16" in ss2d.describe(2, 192, 256, 256, 16)  # segmented either way
    assert "lanes_per_seq=32" in ss2d.describe(1, 11, 96, 100, 16)    # segmented, 128 steps left


def test_describe_backward_plan():
    # the backward cuts long maps into segments when its channel blocks alone give
    # fewer than 1536 workgroups, and pairs channel blocks (one segment) while that
    # still leaves 768 workgroups
    def plan(*a):
        f = dict(kv.split("=") for kv in ss2d.describe(*a).split())
        return int(f["backward_segments"]), int(f["backward_blocks_per_workgroup"])
    assert plan(32, 192, 56, 56, 16, ss2d.SS2D_F32) == (1, 2)    # 1536 blocks
    assert plan(32, 768, 14, 14, 16, ss2d.SS2D_F32) == (1, 2)
    assert plan(64, 384, 28, 28, 16, ss2d.SS2D_BF16) == (1, 2)   # bf16 pairs too
    assert plan(2, 192, 256, 256, 16, ss2d.SS2D_F32) == (16, 1)  # 96 blocks: 16 segments
    assert plan(1, 192, 56, 56, 16, ss2d.SS2D_F32) == (5, 1)
    assert plan(1, 16, 8, 8, 16, ss2d.SS2D_F32) == (1, 1)        # one chunk: nothing to cut
    assert plan(16, 192, 56, 56, 16, ss2d.SS2D_F32) == (1, 1)    # 768 blocks fill the chip once: whole


def test_describe_bidir_backward_plan():
    # the two-path backward over L = H*W tokens: two walks per batch element
    def plan(*a):
        f = dict(kv.split("=") for kv in ss2d.describe(*a).split())
        return int(f["bidir_backward_segments"]), int(f["bidir_backward_blocks_per_workgroup"])
    assert plan(32, 192, 56, 56, 16, ss2d.SS2D_F32) == (1, 1)    # 768 blocks
    assert plan(64, 192, 56, 56, 16, ss2d.SS2D_F32) == (1, 2)    # 1536 blocks: pairs
    assert plan(2, 192, 256, 256, 16, ss2d.SS2D_F32) == (32, 1)  # 48 blocks: 32 segments


# fake, well-aligned, non-overlapping addresses (never dereferenced: validation fails first)
BASE = 1 << 40
X, DT, AL, BI, BS, CS, DS, Y = (BASE + i * (1 << 34) for i in range(8))


def _call(x=X, dt=DT, al=AL, bi=BI, bs=BS, cs=CS, ds=DS, y=Y, B=2, D=3, H=4, W=5, N=16, dtype=0):
    return ss2d.ss2d_forward(x, dt, al, bi, bs, cs, ds, y, B, D, H, W, N, dtype, None)


@pytest.mark.parametrize("which", range(8))
def test_null_pointer(which):
    args = [X, DT, AL, BI, BS, CS, DS, Y]
    args[which] = None
    assert _call(*args) == -1


@pytest.mark.parametrize("shape", [(0, 3, 4, 5), (2, 0, 4, 5), (2, 3, 0, 5), (2, 3, 4, 0), (-1, 3, 4, 5),
                                   (1, 1, 1 << 31, 1 << 31), (1 << 40, 1 << 20, 8, 8),
                                   (1, 1, 1 << 13, 1 << 12)])  # H*W = 2^25: past the 32-bit row offsets
def test_bad_shape(shape):
    B, D, H, W = shape
    assert _call(B=B, D=D, H=H, W=W) == -2


@pytest.mark.parametrize("N", [0, -1, 257, 1 << 20])
def test_unsupported_state_size(N):
    assert _call(N=N) == -3


@needs_no_device
@pytest.mark.parametrize("N", [1, 17, 64, 256])
def test_large_state_sizes_are_accepted(N):
    assert _call(N=N) == -7


@pytest.mark.parametrize("dtype", [2, -1, 7])
def test_bad_dtype(dtype):
    assert _call(dtype=dtype) == -4


def test_output_aliasing_an_input():
    assert _call(y=X) == -5
    assert _call(y=DT + 64) == -5
    assert _call(y=CS - 16) == -5   # y's range reaches into Cs
    assert _call(y=AL) == -5


def test_misaligned_pointers():
    # only element misalignment is an error
    assert _call(x=X + 2) == -6
    assert _call(al=AL + 1) == -6
    assert _call(x=X + 1, dtype=1) == -6
    assert _call(y=Y + 3, H=4, W=4) == -6


@needs_no_device
def test_element_aligned_bases_are_accepted():
    """Bases aligned to their element but not to 16 (fp32) / 8 (bf16) bytes take the
    scalar path instead of being rejected."""
    assert _call(x=X + 4, dtype=1, H=4, W=4) == -7
    assert _call(dt=DT + 4, H=4, W=4) == -7
    assert _call(y=Y + 8, bs=BS + 4, H=8, W=8) == -7


# the two-path scan: x (B, D, L), per-path tensors with two slots
def _bidir(x=X, dt=DT, al=AL, bi=BI, bs=BS, cs=CS, ds=DS, y=Y, B=2, D=3, L=20, N=16, dtype=0):
    return ss2d.ss2d_bidir_forward(x, dt, al, bi, bs, cs, ds, y, B, D, L, N, dtype, None)


def test_bidir_validation():
    for i in range(8):
        args = [X, DT, AL, BI, BS, CS, DS, Y]
        args[i] = None
        assert _bidir(*args) == -1
    assert _bidir(L=0) == -2
    assert _bidir(N=0) == -3
    assert _bidir(N=257) == -3
    assert _bidir(dtype=3) == -4
    assert _bidir(y=DT + 8) == -5
    assert _bidir(x=X + 2) == -6


@needs_no_device
def test_bidir_valid_calls_without_device_report_no_device():
    assert _bidir() == -7
    assert _bidir(N=256, dtype=1) == -7
    # the (B, 2, D, L) dt ends where a (B, 4, D, L) one would still run on: y may start there
    assert _bidir(y=DT + 2 * 2 * 3 * 20 * 4) == -7


@needs_no_device
def test_forward_lanes_call():
    L = ss2d.lib()
    args = (X, DT, AL, BI, BS, CS, DS, Y, 2, 3, 4, 5, 16, 0)
    assert L.ss2d_forward_lanes(*args, 48, None) == -2
    for lanes in (0, 16, 32, 64):
        assert L.ss2d_forward_lanes(*args, lanes, None) == -7


@needs_no_device
def test_measure_peaks_validates_before_touching_a_device():
    L = ss2d.lib()
    p = ss2d.Peaks()
    assert L.ss2d_measure_peaks(None, 1 << 20, None) == -1
    for bad in (0, 1000, (1 << 20) + 4, (65 << 30)):
        assert L.ss2d_measure_peaks(ctypes.byref(p), bad, None) == -2, bad
    assert L.ss2d_measure_peaks(ctypes.byref(p), 1 << 20, None) == -7  # no GPU in this container


@needs_no_device
def test_valid_call_without_device_reports_no_device():
    assert _call() == -7


# the projection entry points: same fake addresses, weights in their own slots
WX, WDT = BASE + 8 * (1 << 34), BASE + 9 * (1 << 34)


def _proj(x=X, wx=WX, wdt=WDT, dt=DT, bs=BS, cs=CS, B=2, D=3, H=4, W=5, N=16, R=2, dtype=0):
    return ss2d.ss2d_project(x, wx, wdt, dt, bs, cs, B, D, H, W, N, R, dtype, None)


def _fromx(x=X, wx=WX, wdt=WDT, al=AL, bi=BI, ds=DS, y=Y, B=2, D=3, H=4, W=5, N=16, R=2, dtype=0):
    return ss2d.ss2d_forward_from_x(x, wx, wdt, al, bi, ds, y, B, D, H, W, N, R, dtype, None)


@pytest.mark.parametrize("which", range(6))
def test_project_null_pointer(which):
    args = [X, WX, WDT, DT, BS, CS]
    args[which] = None
    assert _proj(*args) == -1


@pytest.mark.parametrize("which", range(7))
def test_forward_from_x_null_pointer(which):
    args = [X, WX, WDT, AL, BI, DS, Y]
    args[which] = None
    assert _fromx(*args) == -1


@pytest.mark.parametrize("call", [_proj, _fromx])
def test_projection_rank_and_row_limits(call):
    assert call(R=0) == -2
    assert call(R=-3) == -2
    assert call(N=16, R=33) == -2     # 2 * (33 + 32) = 130 rows > 128
    assert call(N=1, R=63) == -2      # 2 * (63 + 2) = 130
    assert call(N=17) == -3           # the projections take N <= 16
    assert call(dtype=3) == -4
    assert call(B=0) == -2


def test_projection_aliasing_and_alignment():
    assert _proj(dt=X) == -5
    assert _proj(bs=CS) == -5          # two outputs on one buffer
    assert _proj(cs=WX + 64) == -5     # an output over a weight
    assert _proj(wx=WX + 2) == -6
    assert _proj(x=X + 1, dtype=1) == -6
    assert _fromx(y=X) == -5
    assert _fromx(y=WDT) == -5
    assert _fromx(wdt=WDT + 1) == -6
    assert _fromx(x=X + 2) == -6


@needs_no_device
def test_projection_valid_calls_without_device_report_no_device():
    assert _proj() == -7
    assert _proj(N=16, R=32) == -7     # exactly 128 rows is allowed
    assert _fromx() == -7
    assert _fromx(x=X + 4, H=4, W=4) == -7   # element-aligned x takes the scalar paths


# the channel-last epilogue
GM, BT, OUT = BASE + 10 * (1 << 34), BASE + 11 * (1 << 34), BASE + 12 * (1 << 34)


def _epi(y=X, g=GM, b=BT, eps=1e-5, norm=1, out=OUT, B=2, D=3, H=4, W=5, dtype=0):
    return ss2d.ss2d_channel_last(y, g, b, eps, norm, out, B, D, H, W, dtype, None)


def test_channel_last_validation():
    assert _epi(y=None) == -1
    assert _epi(out=None) == -1
    assert _epi(D=4097) == -2
    assert _epi(norm=2) == -2
    assert _epi(eps=-1.0) == -2
    assert _epi(eps=float("nan")) == -2
    assert _epi(eps=float("inf")) == -2
    assert _epi(dtype=5) == -4
    assert _epi(H=0) == -2
    assert _epi(out=X + 8) == -5
    assert _epi(out=GM) == -5
    assert _epi(y=X + 1, dtype=1) == -6
    assert _epi(g=GM + 2) == -6


@needs_no_device
def test_channel_last_valid_calls_without_device_report_no_device():
    assert _epi(out=OUT + 4, D=8) == -7             # element alignment is enough (then: no device)
    assert _epi() == -7
    assert _epi(g=None, b=None) == -7               # scale and shift are optional
    assert _epi(norm=0, eps=-1.0) == -7             # eps is unused without the normalisation
    assert _epi(D=4096) == -7


# the backward
GRAD = [BASE + (13 + i) * (1 << 34) for i in range(8)]  # dy, then the seven outputs


def _bwd(ptrs=None, B=2, D=3, H=4, W=5, N=16, dtype=0):
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD if ptrs is None else ptrs
    return ss2d.ss2d_backward(*p, B, D, H, W, N, dtype, None)


def test_backward_validation():
    for i in range(15):
        p = [X, DT, AL, BI, BS, CS, DS] + GRAD
        p[i] = None
        assert _bwd(p) == -1, i
    assert _bwd(dtype=2) == -4
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD
    p[0] = X + 1                          # bf16 tensors need 2-byte alignment
    assert _bwd(p, dtype=1) == -6
    assert _bwd(N=0) == -3
    assert _bwd(N=257) == -3              # up to 256 states, in passes of 16
    assert _bwd(W=0) == -2
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD
    p[8] = X                              # dx on top of x
    assert _bwd(p) == -5
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD
    p[13] = p[12]                         # dCs on top of dBs
    assert _bwd(p) == -5
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD
    p[10] = GRAD[3] + 2                   # dA_log misaligned
    assert _bwd(p) == -6


def _bidir_bwd(ptrs=None, B=2, D=3, L=20, N=16, dtype=0):
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD if ptrs is None else ptrs
    return ss2d.ss2d_bidir_backward(*p, B, D, L, N, dtype, None)


def test_bidir_backward_validation():
    for i in range(15):
        p = [X, DT, AL, BI, BS, CS, DS] + GRAD
        p[i] = None
        assert _bidir_bwd(p) == -1, i
    assert _bidir_bwd(dtype=2) == -4
    assert _bidir_bwd(N=0) == -3
    assert _bidir_bwd(N=257) == -3
    assert _bidir_bwd(L=0) == -2
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD
    p[8] = X                              # dx on top of x
    assert _bidir_bwd(p) == -5
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD
    p[9] = DT + 4                         # ddt inside dt
    assert _bidir_bwd(p) == -5
    p = [X, DT, AL, BI, BS, CS, DS] + GRAD
    p[0] = X + 1                          # bf16 tensors need 2-byte alignment
    assert _bidir_bwd(p, dtype=1) == -6


@needs_no_device
def test_bidir_backward_valid_calls_without_device_report_no_device():
    assert _bidir_bwd() == -7
    assert _bidir_bwd(N=40, dtype=1) == -7


@needs_no_device
def test_backward_valid_calls_without_device_report_no_device():
    assert _bwd(dtype=1) == -7            # bf16 is accepted
    assert _bwd() == -7
    assert _bwd(N=17) == -7               # more than 16 states run in passes
    assert _bwd(N=256, dtype=1) == -7


# the no-allocation forward: same validation, plus the static array's limit
def _noalloc(x=X, dt=DT, al=AL, bi=BI, bs=BS, cs=CS, ds=DS, y=Y, B=2, D=3, H=4, W=5, N=16, dtype=0):
    return ss2d.ss2d_forward_noalloc(x, dt, al, bi, bs, cs, ds, y, B, D, H, W, N, dtype, None)


def test_noalloc_validation_and_limit():
    assert _noalloc(x=None) == -1
    assert _noalloc(H=0) == -2
    assert _noalloc(N=257) == -3
    assert _noalloc(dtype=9) == -4
    assert _noalloc(y=X) == -5
    assert _noalloc(x=X + 2) == -6
    # two fp32 planes of 64 x 384 x 28 x 28 (bf16 output) = 154 MB > 128 MiB: refused before any device work
    assert _noalloc(B=64, D=384, H=28, W=28, dtype=1) == -9
    assert _noalloc(B=64, D=192, H=56, W=56) == -9       # one fp32 plane of 64 x 192 x 3136 is 154 MB
    assert "128 MiB" in open(HEADER).read()


@needs_no_device
def test_noalloc_valid_calls_without_device_report_no_device():
    assert _noalloc() == -7
    assert _noalloc(B=32, D=192, H=56, W=56) == -7       # VMamba-T stage-1 fp32: 77 MB
    assert _noalloc(B=2, D=192, H=256, W=256) == -7      # segmented 256 x 256 map: 107 MB
