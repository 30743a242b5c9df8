"""GPU parity of the two-path scan's backward (ss2d_bidir_backward) against the
float64 oracle oracle/bidir.py's bidir_backward_f64, gradient by gradient,
through the C ABI.  Tolerances as for ss2d_backward: relative L2 <= 1e-5 for the
per-element gradients and 1e-4 for the per-channel parameter gradients (sums of
up to ~10^5 terms); bf16 storage holds the per-element gradients to 1e-2 (their
output rounding) and the fp32 parameter gradients to 1e-4.
"""
import numpy as np
import pytest

from oracle import bidir
import ss2d_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = {"dx": 1e-5, "ddt": 1e-5, "dBs": 1e-5, "dCs": 1e-5, "dA_log": 1e-4, "ddt_bias": 1e-4, "dDs": 1e-4}


def _run(B, D, L, N, seed, dtype="f32", element=None):
    """GPU gradients against the oracle; element: check batch element 0 alone (the
    per-element gradients; the oracle then runs on that element only)."""
    inp = ss2d_inputs.bidir_random(B, D, L, N, seed=seed, dtype=dtype)
    rng = np.random.default_rng(seed + 3)
    dy = rng.standard_normal((B, D, L)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        dy = ss2d_inputs.round_to_bf16(dy)
    d = {k: (torch.from_numpy(v).to(tdt) if k in ("x", "dt", "Bs", "Cs") else torch.from_numpy(v)).cuda()
         for k, v in inp.items()}
    import selective_scan_crossscan_amd as ss2d
    got = ss2d.bidir_backward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"],
                              torch.from_numpy(dy).to(tdt).cuda())
    torch.cuda.synchronize()
    keys = ("dx", "ddt", "dBs", "dCs") if element else tuple(TOL)
    if element:
        inp = {k: (v[:1] if k in ("x", "dt", "Bs", "Cs") else v) for k, v in inp.items()}
        dy = dy[:1]
    ref = bidir.bidir_backward_f64(**inp, dy=dy)
    for k in keys:
        g = got[k][:1] if element else got[k]
        g = g.double().cpu().numpy()
        assert g.shape == ref[k].shape, k
        e = float(np.linalg.norm(g - ref[k]) / max(np.linalg.norm(ref[k]), 1e-300))
        print(k, f"{e:.2e}", flush=True)
        tol = 1e-2 if dtype == "bf16" and k in ("dx", "ddt", "dBs", "dCs") else TOL[k]
        assert e <= tol, (k, e)
    return got


# (B, D, L, N, dtype): one-element accesses (L % 4 != 0), ragged chunks with D past
# the channel block, a sequence cut into segments, passes of 16 states (two, and
# three with a middle one), bf16 storage, one token, one state
SHAPES = [(2, 5, 37, 16, "f32"), (2, 20, 300, 16, "f32"), (1, 16, 2048, 16, "f32"), (2, 20, 200, 24, "bf16"),
          (1, 17, 130, 40, "f32"), (2, 9, 64, 7, "bf16"), (1, 3, 1, 16, "f32"), (3, 33, 11, 1, "f32")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bidir_backward_matches_oracle(shape):
    *dims, dtype = shape
    print(f"[bidir backward] {shape}", flush=True)
    _run(*dims, seed=sum(dims), dtype=dtype)


def test_bidir_backward_stage1_tokens_batch_element():
    # the token count of the VMamba-T stage-1 map (32 x 192 x 3136, N = 16), the
    # workload the two-path bench runs; batch element 0 against the oracle
    import selective_scan_crossscan_amd as ss2d
    f = dict(kv.split("=") for kv in ss2d.describe(32, 192, 56, 56, 16).split())
    assert (f["bidir_backward_segments"], f["bidir_backward_blocks_per_workgroup"]) == ("1", "1")
    print("[bidir backward] 32x192x3136", flush=True)
    _run(32, 192, 3136, 16, seed=5, element=True)


def test_bidir_backward_is_deterministic():
    a = _run(1, 24, 100, 16, seed=9)
    b = _run(1, 24, 100, 16, seed=9)
    for k in a:
        assert torch.equal(a[k], b[k]), k
