"""GPU parity of the projection path (ss2d_project, ss2d_forward_from_x) against
the float64 oracle in oracle/projection.py, element by element.

Tolerances.
  * Projections, fp32 storage: any fp32 evaluation of a sum of n products of
    fp32 numbers is within n*u*sum|w||x| of the exact value (u = 2^-24; Higham's
    bound gamma_n, n*u << 1), plus u*|value| for the final rounding.  dt is two
    such sums in a row, so its bound uses n = D + R + 2 over the absolute
    contraction |W_dt| |W_x| |x|.  The oracle computes those absolute sums.
  * bf16 storage adds the final rounding to bfloat16: 2^-8 |value|.
  * y: the forward's bars (fp32: rel-L2 <= 1e-5 and max|err| <= 1e-4 max|y|;
    bf16: rel-L2 <= 2e-2).
Every call goes through the C ABI.
"""
import numpy as np
import pytest

import oracle
from oracle import projection
import ss2d_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U32 = 2.0 ** -24


def _lib():
    import selective_scan_crossscan_amd as ss2d
    return ss2d


def _dev(inp, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k == "x":
            t = t.to(tdt)
        out[k] = t.cuda()
    return out


def _inputs(B, D, H, W, N, R, dtype="f32", seed=0):
    return ss2d_inputs.generate_projected(ss2d_inputs.Shape("t", B, D, H, W, N, dtype), seed=seed, R=R)


def _check_projection(inp, dtype):
    N = inp["A_log"].shape[1]
    R = inp["dt_projs_weight"].shape[2]
    D = inp["x"].shape[1]
    d = _dev(inp, dtype)
    got = _lib().project(d["x"], d["x_proj_weight"], d["dt_projs_weight"], N)
    torch.cuda.synchronize()
    ref = projection.project(inp["x"], inp["x_proj_weight"], inp["dt_projs_weight"], N)
    mag = projection.project_abs(inp["x"], inp["x_proj_weight"], inp["dt_projs_weight"], N)
    final = 2.0 ** -8 if dtype == "bf16" else U32
    for name, g, r, a, n in zip(("dt", "Bs", "Cs"), got, ref, mag, (D + R + 2, D, D)):
        g = g.double().cpu().numpy()
        assert g.shape == r.shape, name
        bound = 1.01 * (n * U32 * a + final * np.abs(r)) + 1e-30
        err = np.abs(g - r)
        worst = np.unravel_index(np.argmax(err / bound), err.shape)
        assert np.all(err <= bound), (name, worst, g[worst], r[worst], bound[worst])


def _check_forward(inp, dtype):
    d = _dev(inp, dtype)
    y = _lib().forward_from_x(d["x"], d["x_proj_weight"], d["dt_projs_weight"], d["A_log"], d["dt_bias"], d["Ds"])
    torch.cuda.synchronize()
    ref = projection.ss2d_from_x_f64(inp["x"], inp["x_proj_weight"], inp["dt_projs_weight"], inp["A_log"],
                                     inp["dt_bias"], inp["Ds"])
    got = y.double().cpu().numpy()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    if dtype == "bf16":
        assert rel <= 2e-2, rel
    else:
        assert rel <= 1e-5, rel
        assert np.max(np.abs(got - ref)) <= 1e-4 * np.max(np.abs(ref))
    return y


# (B, D, H, W, N, R, dtype): several 16-row tiles and 64-position strips, ragged
# strips (L % 64), L % 4 != 0 (scalar path), D % 16 != 0 (ragged channel step),
# one row tile (N = 1, R = 1), the 128-row maximum, bf16 storage.  D a multiple
# of 32 takes the LDS-staged operands: one workgroup per direction on the small
# maps, both directions per workgroup on the last two (at least 512 strips), with
# a ragged last strip, in both storage types.
SHAPES = [
    (1, 16, 8, 8, 16, 1, "f32"),
    (2, 20, 5, 7, 4, 3, "f32"),
    (1, 64, 9, 12, 16, 2, "f32"),
    (2, 8, 3, 3, 1, 1, "f32"),
    (1, 64, 6, 10, 16, 32, "f32"),
    (1, 33, 7, 9, 16, 5, "f32"),
    (2, 48, 8, 12, 16, 2, "bf16"),
    (1, 20, 5, 7, 3, 2, "bf16"),
    (40, 32, 20, 20, 16, 4, "f32"),
    (64, 64, 12, 20, 16, 4, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_projection_matches_oracle(shape):
    B, D, H, W, N, R, dtype = shape
    print(f"[projection] {shape}", flush=True)
    _check_projection(_inputs(B, D, H, W, N, R, dtype, seed=sum(shape[:6])), dtype)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_from_x_matches_oracle(shape):
    B, D, H, W, N, R, dtype = shape
    print(f"[from_x] {shape}", flush=True)
    _check_forward(_inputs(B, D, H, W, N, R, dtype, seed=1 + sum(shape[:6])), dtype)


def test_forward_from_x_segmented_map():
    # 64 x 64 with two batches of 16 channels: a segmented plan (carry pass and
    # per-direction launches) reading the caller-made transposed copy
    assert "segments=1 " not in _lib().describe(1, 16, 64, 64, 16, 0)
    _check_forward(_inputs(1, 16, 64, 64, 16, 1, "f32", seed=5), "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_from_x_equals_forward_on_projected_inputs(dtype):
    # rank 9 (past the low-rank input's limit of 8): same projections, same scan
    # arithmetic, so reading x through the transposed copy must not change a bit
    inp = _inputs(2, 32, 12, 20, 16, 9, dtype, seed=9)
    d = _dev(inp, dtype)
    ss2d = _lib()
    y1 = ss2d.forward_from_x(d["x"], d["x_proj_weight"], d["dt_projs_weight"], d["A_log"], d["dt_bias"], d["Ds"])
    dt, Bs, Cs = ss2d.project(d["x"], d["x_proj_weight"], d["dt_projs_weight"], 16)
    y2 = ss2d.forward(d["x"], dt, d["A_log"], d["dt_bias"], Bs, Cs, d["Ds"])
    y3 = ss2d.forward_from_x(d["x"], d["x_proj_weight"], d["dt_projs_weight"], d["A_log"], d["dt_bias"], d["Ds"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1, y3)


# Ranks up to 8 hand the scan the low-rank rows, which forms dt itself (R FMAs per
# channel and step): fused plans with remainder chunks, a prefetched remainder,
# the register-staged path (L % 4 != 0), a segmented plan, bf16, R at the limit.
LOW_RANK = [
    (1, 16, 40, 40, 16, 6, "f32"),   # 1600 steps: 3 chunks and a prefetched 64-step remainder
    (2, 24, 9, 14, 16, 3, "f32"),    # L % 4 != 0: every chunk through the register-staged path
    (1, 32, 28, 28, 16, 8, "bf16"),  # R = 8, bf16, 16 lanes
    (1, 16, 72, 72, 16, 4, "f32"),   # segmented: the carry pass and the per-direction launches
    (2, 40, 14, 14, 7, 5, "f32"),    # one partial chunk, odd N
]


@pytest.mark.parametrize("shape", LOW_RANK, ids=lambda s: "x".join(map(str, s)))
def test_forward_from_x_low_rank_input(shape):
    """The low-rank path against the oracle, and against the forward on the projected
    inputs (dt formed by the projection kernel) to the forward's tolerances."""
    B, D, H, W, N, R, dtype = shape
    print(f"[from_x low rank] {shape} {_lib().describe(B, D, H, W, N, 1 if dtype == 'bf16' else 0)}", flush=True)
    inp = _inputs(B, D, H, W, N, R, dtype, seed=R + H)
    y = _check_forward(inp, dtype).double().cpu().numpy()
    d = _dev(inp, dtype)
    ss2d = _lib()
    dt, Bs, Cs = ss2d.project(d["x"], d["x_proj_weight"], d["dt_projs_weight"], N)
    y2 = ss2d.forward(d["x"], dt, d["A_log"], d["dt_bias"], Bs, Cs, d["Ds"])
    torch.cuda.synchronize()
    y2 = y2.double().cpu().numpy()
    rel = float(np.linalg.norm(y - y2) / np.linalg.norm(y2))
    print(f"[from_x low rank] vs forward on projected inputs: rel_l2 {rel:.3e}", flush=True)
    assert rel <= (2e-2 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("cfg", [1, 3], ids=["vmamba_t_stage1", "vmamba_t_stage2_bf16"])
def test_full_size_workload(cfg):
    shape = ss2d_inputs.CONFIGS[cfg]
    print(f"[full] {shape}", flush=True)
    inp = ss2d_inputs.generate_projected(shape, seed=0)
    _check_projection(inp, shape.dtype)
    _check_forward(inp, shape.dtype)


def test_rejects_too_many_rows():
    ss2d = _lib()
    x = torch.zeros((1, 8, 4, 4), device="cuda")
    with pytest.raises(ss2d.SS2DError) as e:
        ss2d.project(x, torch.zeros((4, 65 + 32, 8), device="cuda"), torch.zeros((4, 8, 65), device="cuda"), 16)
    assert e.value.code == -2
