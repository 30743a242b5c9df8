"""GPU parity of the backward (ss2d_backward) against the float64 backward oracle
(oracle/backward.py), gradient by gradient, through the C ABI.

Tolerances (fp32 arithmetic, u = 2^-24 ~ 6e-8).  Per-element gradients (dx, ddt,
dBs, dCs) are sums of at most 4N or D products after recurrences whose decays are
below 1, so rounding stays near sqrt(n) u relative: relative L2 <= 1e-5, as for
the forward.  The per-channel parameter gradients (dA_log, ddt_bias, dDs) are sums
over the batch and every step, up to ~10^5 terms with cancellation:
relative L2 <= 1e-4.  bf16 storage (fp32 arithmetic, the oracle reading the same
bf16 inputs): the bf16 outputs carry their rounding, 2^-9 relative per element,
so the per-element gradients are held to relative L2 <= 1e-2; the fp32
parameter gradients keep 1e-4.
"""
import numpy as np
import pytest

from oracle import backward
import ss2d_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = {"dx": 1e-5, "ddt": 1e-5, "dBs": 1e-5, "dCs": 1e-5, "dA_log": 1e-4, "ddt_bias": 1e-4, "dDs": 1e-4}


def _run(B, D, H, W, N, seed, a_log="random", dtype="f32", a_log_value=None):
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=seed, a_log=a_log, dtype=dtype)
    if a_log_value is not None:
        inp["A_log"][:] = a_log_value
    rng = np.random.default_rng(seed + 7)
    dy = rng.standard_normal((B, D, H, W)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        dy = ss2d_inputs.round_to_bf16(dy)
    d = {k: (torch.from_numpy(v).to(tdt) if k in ("x", "dt", "Bs", "Cs") else torch.from_numpy(v)).cuda()
         for k, v in inp.items()}
    import selective_scan_crossscan_amd as ss2d
    got = ss2d.backward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"],
                        torch.from_numpy(dy).to(tdt).cuda())
    torch.cuda.synchronize()
    ref = backward.ss2d_backward_f64(**inp, dy=dy)
    errs = {}
    for k, r in ref.items():
        g = got[k].double().cpu().numpy()
        assert g.shape == r.shape, k
        errs[k] = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        tol = 1e-2 if dtype == "bf16" and k in ("dx", "ddt", "dBs", "dCs") else TOL[k]
        assert e <= tol, (k, e)
    return got


# (B, D, H, W, N): one segment, D past the 16-channel block, several segments with a
# ragged last one, H = 1 and W = 1 (walks of one column or one row), N < 16
SHAPES = [(1, 2, 2, 3, 3), (2, 5, 3, 7, 16), (1, 17, 8, 9, 7), (2, 16, 16, 16, 16), (1, 3, 1, 37, 16),
          (1, 3, 37, 1, 16), (1, 20, 12, 20, 16), (3, 33, 5, 11, 1)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_matches_oracle(shape):
    print(f"[backward] {shape}", flush=True)
    _run(*shape, seed=sum(shape))


def test_backward_at_stage1_size_per_batch():
    # one batch of the VMamba-T stage-1 shape (D = 192, 56 x 56, N = 16), S4D A_log
    print("[backward] 1x192x56x56", flush=True)
    _run(1, 192, 56, 56, 16, seed=1, a_log="s4d")


def test_backward_is_deterministic():
    a = _run(1, 24, 9, 10, 16, seed=3)
    b = _run(1, 24, 9, 10, 16, seed=3)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("shape", [(1, 5, 6, 7, 16), (2, 20, 12, 11, 9)], ids=lambda s: "x".join(map(str, s)))
def test_backward_bf16_storage(shape):
    print(f"[backward bf16] {shape}", flush=True)
    _run(*shape, seed=sum(shape) + 1, dtype="bf16")


def test_backward_bf16_at_stage2_size_per_batch():
    # one batch of the VMamba-T stage-2 bf16 shape (D = 384, 28 x 28, N = 16)
    print("[backward bf16] 1x384x28x28", flush=True)
    _run(1, 384, 28, 28, 16, seed=2, a_log="s4d", dtype="bf16")


def _plan(B, D, H, W, N, dtype=0):
    import selective_scan_crossscan_amd as ss2d
    desc = ss2d.describe(B, D, H, W, N, dtype)
    return {k: int(desc.split(k + "=")[1].split()[0]) for k in ("backward_segments", "backward_blocks_per_workgroup")}


def _segments(B, D, H, W, N):
    return _plan(B, D, H, W, N)["backward_segments"]


# (B, D, H, W, N, dtype): maps cut into segments -- two segments of four chunks,
# three with a ragged last segment, a ragged last chunk and a ragged channel block,
# four segments over two batches, bf16 with N < 16; planes too large for one LDS
# tile, whose transposes of x and dy go in 64 x 64 tiles with ragged edges (W a
# multiple of 4 or not)
SEG_SHAPES = [(1, 16, 32, 32, 16, "f32"), (1, 20, 40, 41, 16, "f32"), (2, 16, 48, 48, 16, "f32"),
              (1, 16, 33, 37, 5, "bf16"), (1, 3, 96, 160, 16, "f32"), (1, 2, 100, 130, 16, "f32")]


@pytest.mark.parametrize("shape", SEG_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_segmented_matches_oracle(shape):
    *dims, dtype = shape
    assert _segments(*dims) > 1
    print(f"[backward segmented] {shape}", flush=True)
    _run(*dims, seed=sum(dims) + 3, dtype=dtype)


def test_backward_segmented_slow_decay():
    # A = -exp(-4): states and adjoints keep most of their size across a segment,
    # so the chained entering state and adjoint carry real weight
    assert _segments(1, 16, 40, 41, 16) == 3
    print("[backward segmented, slow decay] 1x16x40x41", flush=True)
    _run(1, 16, 40, 41, 16, seed=11, a_log_value=-4.0)


@pytest.mark.parametrize("cfg,segmented", [(1, False), (4, True)], ids=["vmamba_t_stage1", "highres_256"])
def test_backward_full_size_sampled_channels(cfg, segmented):
    # a full-size shape in the plan the benchmark times (stage 1: one workgroup
    # walks all 25 chunks; 256 x 256: 16 segments); the oracle recomputes three
    # channels on their own (every gradient but dBs and dCs, which sum over all
    # channels, depends only on its channel's inputs)
    shape = ss2d_inputs.CONFIGS[cfg]
    B, D, H, W, N = shape.B, shape.D, shape.H, shape.W, shape.N
    assert (_segments(B, D, H, W, N) > 1) == segmented
    print(f"[backward full size] {shape}", flush=True)
    inp = ss2d_inputs.generate(shape, seed=4)
    rng = np.random.default_rng(5)
    dy = rng.standard_normal((B, D, H, W)).astype(np.float32)
    import selective_scan_crossscan_amd as ss2d
    d = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    got = ss2d.backward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"],
                        torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    idx = np.array([0, 77, D - 1])
    per_k = lambda v: v.reshape(4, D, *v.shape[1:])[:, idx].reshape(4 * len(idx), *v.shape[1:])
    sub = dict(x=inp["x"][:, idx], dt=inp["dt"][:, :, idx], A_log=per_k(inp["A_log"]),
               dt_bias=per_k(inp["dt_bias"]), Bs=inp["Bs"], Cs=inp["Cs"], Ds=per_k(inp["Ds"]))
    del inp, d
    ref = backward.ss2d_backward_f64(**sub, dy=dy[:, idx])
    cols = torch.from_numpy(np.concatenate([k * D + idx for k in range(4)]))
    pick = {"dx": got["dx"][:, idx], "ddt": got["ddt"][:, :, idx], "dA_log": got["dA_log"][cols],
            "ddt_bias": got["ddt_bias"][cols], "dDs": got["dDs"][cols]}
    for k, g in pick.items():
        g = g.double().cpu().numpy()
        r = ref[k]
        assert g.shape == r.shape, k
        e = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        print(k, f"{e:.2e}", flush=True)
        assert e <= TOL[k], (k, e)


@pytest.mark.parametrize("cfg,nsp,cpb", [(1, 1, 2), (2, 1, 2), (3, 1, 2), ("2x192x90x90", 16, 1)],
                         ids=["vmamba_t_stage1", "vmamba_t_stage3", "vmamba_t_stage2_bf16", "segmented_2x192x90x90"])
def test_backward_full_size_batch_element(cfg, nsp, cpb):
    # a full-size shape in the plan the benchmark times (two channel blocks per
    # workgroup sharing one dBs/dCs partial), and a 90 x 90 map cut into 16
    # segments as the 256 x 256 map is; the oracle recomputes batch element 0 on its
    # own (its dx, ddt, dBs and dCs depend only on its inputs)
    shape = (ss2d_inputs.CONFIGS[cfg] if isinstance(cfg, int)
             else ss2d_inputs.Shape("segmented", 2, 192, 90, 90, 16, "f32"))
    B, D, H, W, N = shape.B, shape.D, shape.H, shape.W, shape.N
    bf16 = shape.dtype == "bf16"
    assert _plan(B, D, H, W, N, 1 if bf16 else 0) == {"backward_segments": nsp, "backward_blocks_per_workgroup": cpb}
    print(f"[backward full size, batch element 0] {shape}", flush=True)
    inp = ss2d_inputs.generate(shape, seed=6)
    rng = np.random.default_rng(7)
    dy = rng.standard_normal((B, D, H, W)).astype(np.float32)
    tdt = torch.bfloat16 if bf16 else torch.float32
    if bf16:
        dy = ss2d_inputs.round_to_bf16(dy)
    import selective_scan_crossscan_amd as ss2d
    d = {k: (torch.from_numpy(v).to(tdt) if k in ("x", "dt", "Bs", "Cs") else torch.from_numpy(v)).cuda()
         for k, v in inp.items()}
    got = ss2d.backward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"],
                        torch.from_numpy(dy).to(tdt).cuda())
    torch.cuda.synchronize()
    sub = {k: (v[:1] if k in ("x", "dt", "Bs", "Cs") else v) for k, v in inp.items()}
    ref = backward.ss2d_backward_f64(**sub, dy=dy[:1])
    for k in ("dx", "ddt", "dBs", "dCs"):
        g = got[k][:1].double().cpu().numpy()
        e = float(np.linalg.norm(g - ref[k]) / np.linalg.norm(ref[k]))
        print(k, f"{e:.2e}", flush=True)
        assert e <= (1e-2 if bf16 else TOL[k]), (k, e)


# (B, D, H, W, N, dtype): more than 16 states run in passes of 16 states whose
# du, ddt and ddt_bias add up in pass order: two passes (16 + 1), three with a
# middle pass, bf16, a segmented map, and one-element accesses (L % 4 != 0)
LARGE_N = [(1, 20, 12, 11, 17, "f32"), (2, 16, 16, 16, 40, "f32"), (1, 20, 12, 12, 24, "bf16"),
           (1, 16, 32, 32, 20, "f32"), (1, 5, 7, 9, 33, "f32")]


@pytest.mark.parametrize("shape", LARGE_N, ids=lambda s: "x".join(map(str, s)))
def test_backward_large_state(shape):
    *dims, dtype = shape
    print(f"[backward large state] {shape}", flush=True)
    _run(*dims, seed=sum(dims) + 13, dtype=dtype)


def _check_batch_element_and_channels(shape, idx, seed):
    """Full GPU backward of `shape` (storage type as the shape says); the oracle on batch
    element 0 (dx, ddt, dBs, dCs) and on the channels `idx` alone (dA_log, ddt_bias, dDs,
    summed over the batch).  bf16 storage: the per-element gradients to 1e-2 (their
    output rounding), the fp32 parameter gradients as for fp32."""
    B, D, H, W, N = shape.B, shape.D, shape.H, shape.W, shape.N
    bf16 = shape.dtype == "bf16"
    inp = ss2d_inputs.generate(shape, seed=seed, a_log="s4d")
    rng = np.random.default_rng(seed + 1)
    dy = rng.standard_normal((B, D, H, W)).astype(np.float32)
    tdt = torch.bfloat16 if bf16 else torch.float32
    if bf16:
        dy = ss2d_inputs.round_to_bf16(dy)
    import selective_scan_crossscan_amd as ss2d
    d = {k: (torch.from_numpy(v).to(tdt) if k in ("x", "dt", "Bs", "Cs") else torch.from_numpy(v)).cuda()
         for k, v in inp.items()}
    got = ss2d.backward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"],
                        torch.from_numpy(dy).to(tdt).cuda())
    torch.cuda.synchronize()
    sub = {k: (v[:1] if k in ("x", "dt", "Bs", "Cs") else v) for k, v in inp.items()}
    ref = backward.ss2d_backward_f64(**sub, dy=dy[:1])
    for k in ("dx", "ddt", "dBs", "dCs"):
        g = got[k][:1].double().cpu().numpy()
        e = float(np.linalg.norm(g - ref[k]) / np.linalg.norm(ref[k]))
        print(k, f"{e:.2e}", flush=True)
        assert e <= (1e-2 if bf16 else TOL[k]), (k, e)
    idx = np.asarray(idx)
    per_k = lambda v: v.reshape(4, D, *v.shape[1:])[:, idx].reshape(4 * len(idx), *v.shape[1:])
    sub = dict(x=inp["x"][:, idx], dt=inp["dt"][:, :, idx], A_log=per_k(inp["A_log"]),
               dt_bias=per_k(inp["dt_bias"]), Bs=inp["Bs"], Cs=inp["Cs"], Ds=per_k(inp["Ds"]))
    ref = backward.ss2d_backward_f64(**sub, dy=dy[:, idx])
    cols = torch.from_numpy(np.concatenate([k * D + idx for k in range(4)]))
    for k in ("dA_log", "ddt_bias", "dDs"):
        g = got[k][cols].double().cpu().numpy()
        e = float(np.linalg.norm(g - ref[k]) / np.linalg.norm(ref[k]))
        print(k, f"{e:.2e}", flush=True)
        assert e <= TOL[k], (k, e)


def test_backward_large_state_at_stage1_size():
    # the VMamba-T stage-1 shape at N = 64: four passes, each with two channel
    # blocks per workgroup, checked on batch element 0 and three channels
    shape = ss2d_inputs.Shape("vmamba_t_stage1_n64", 32, 192, 56, 56, 64, "f32")
    assert _plan(32, 192, 56, 56, 64) == {"backward_segments": 1, "backward_blocks_per_workgroup": 2}
    print(f"[backward large state, full size] {shape}", flush=True)
    _check_batch_element_and_channels(shape, [0, 77, 191], seed=21)


@pytest.mark.parametrize("dims,dtype", [((32, 192, 16, 16, 5), "f32"), ((28, 200, 16, 16, 16), "f32"),
                                        ((28, 200, 12, 16, 7), "bf16")],
                         ids=["N5", "D200_odd_blocks", "bf16_D200_N7"])
def test_backward_two_blocks_edge_cases(dims, dtype):
    # two channel blocks per workgroup with N < 16, and with an odd number of
    # 16-channel blocks (D = 200: the last workgroup's second block lies past D),
    # in both storage types
    B, D, H, W, N = dims
    assert _plan(B, D, H, W, N, 1 if dtype == "bf16" else 0) == {"backward_segments": 1,
                                                                  "backward_blocks_per_workgroup": 2}
    print(f"[backward two blocks] {dims} {dtype}", flush=True)
    _check_batch_element_and_channels(ss2d_inputs.Shape("t", B, D, H, W, N, dtype), [0, 17, D - 1],
                                      seed=sum(dims))


def _offset_copy(t):
    """t's values in a buffer that starts one element past an aligned base."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("dims,dtype", [((2, 20, 12, 12, 16), "f32"), ((1, 16, 32, 32, 16), "f32"),
                                        ((2, 20, 12, 12, 7), "bf16")],
                         ids=["whole", "segmented", "bf16"])
def test_backward_element_aligned_bases(dims, dtype):
    # L a multiple of 4: aligned inputs take the kernels' 16-byte (8-byte bf16)
    # accesses, inputs one element past an aligned base the one-element accesses;
    # both add in the same order, so the gradients are identical, and they match
    # the oracle
    B, D, H, W, N = dims
    print(f"[backward element-aligned bases] {dims} {dtype}", flush=True)
    got = _run(B, D, H, W, N, seed=sum(dims) + 5, dtype=dtype)
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=sum(dims) + 5, a_log="random", dtype=dtype)
    rng = np.random.default_rng(sum(dims) + 5 + 7)
    dy = rng.standard_normal((B, D, H, W)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        dy = ss2d_inputs.round_to_bf16(dy)
    d = {k: (torch.from_numpy(v).to(tdt) if k in ("x", "dt", "Bs", "Cs") else torch.from_numpy(v)).cuda()
         for k, v in inp.items()}
    off = {k: _offset_copy(d[k]) for k in ("x", "dt", "Bs", "Cs")}
    assert all(t.data_ptr() % 16 != 0 for t in off.values())
    import selective_scan_crossscan_amd as ss2d
    again = ss2d.backward(off["x"], off["dt"], d["A_log"], d["dt_bias"], off["Bs"], off["Cs"], d["Ds"],
                          _offset_copy(torch.from_numpy(dy).to(tdt).cuda()))
    torch.cuda.synchronize()
    for k in got:
        assert torch.equal(got[k], again[k]), k
