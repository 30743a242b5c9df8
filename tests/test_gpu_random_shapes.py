"""Seeded sweeps of small random shapes through every entry point, against the
oracles, with the tolerances of the dedicated tests: the forward (fp32 rel-L2
<= 1e-5 and max |err| <= 1e-4 max|y|; bf16 rel-L2 <= 2e-2), the forward from x
(the same), the epilogue (1e-5 (1 + |out|)), the backward (rel-L2 <= 1e-5 per
element gradient, 1e-2 for bf16 storage, 1e-4 for the parameter sums).  Shapes mix odd D, H, W, N and
rank R, L % 4 != 0, D off the channel blocks, and both storage types.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as obwd
from oracle import epilogue as oepi
from oracle import projection as oproj
import ss2d_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        B = int(rng.integers(1, 3))
        D = int(rng.integers(1, 41))
        H = int(rng.integers(1, 23))
        W = int(rng.integers(1, 23))
        N = int(rng.choice([1, 2, 5, 8, 13, 16]))
        dtype = "bf16" if rng.random() < 0.3 else "f32"
        out.append((B, D, H, W, N, dtype))
    return out


def _lib():
    import selective_scan_crossscan_amd as ss2d
    return ss2d


def _check_y(got, ref, dtype):
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    if dtype == "bf16":
        assert rel <= 2e-2, rel
    else:
        assert rel <= 1e-5, rel
        assert np.max(np.abs(got - ref)) <= 1e-4 * max(np.max(np.abs(ref)), 1e-30)


@pytest.mark.parametrize("shape", _shapes(101, 16), ids=lambda s: "x".join(map(str, s)))
def test_forward_random(shape):
    B, D, H, W, N, dtype = shape
    print(f"[random forward] {shape}", flush=True)
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=B + D + H + W + N, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {k: (torch.from_numpy(v).to(tdt) if k in ("x", "dt", "Bs", "Cs") else torch.from_numpy(v)).cuda()
         for k, v in inp.items()}
    y = _lib().forward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"])
    torch.cuda.synchronize()
    _check_y(y.double().cpu().numpy(), oracle.ss2d_inputs_f64(inp), dtype)


@pytest.mark.parametrize("shape", _shapes(202, 12), ids=lambda s: "x".join(map(str, s)))
def test_forward_from_x_random(shape):
    B, D, H, W, N, dtype = shape
    rng = np.random.default_rng(D * 7 + N)
    R = int(rng.integers(1, 64 - 2 * N + 1)) if 2 * N < 64 else 1
    R = min(R, 12)
    print(f"[random from_x] {shape} R={R}", flush=True)
    inp = ss2d_inputs.generate_projected(ss2d_inputs.Shape("r", B, D, H, W, N, dtype), seed=B + D + H + W, R=R)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {k: (torch.from_numpy(v).to(tdt) if k == "x" else torch.from_numpy(v)).cuda() for k, v in inp.items()}
    y = _lib().forward_from_x(d["x"], d["x_proj_weight"], d["dt_projs_weight"], d["A_log"], d["dt_bias"], d["Ds"])
    torch.cuda.synchronize()
    _check_y(y.double().cpu().numpy(), oproj.ss2d_from_x_f64(**inp), dtype)


@pytest.mark.parametrize("shape", _shapes(303, 12), ids=lambda s: "x".join(map(str, s)))
def test_epilogue_random(shape):
    B, D, H, W, N, dtype = shape
    print(f"[random epilogue] {shape}", flush=True)
    rng = np.random.default_rng(D + H * W)
    y = (rng.standard_normal((B, D, H, W)) * 2 + 1).astype(np.float32)
    if dtype == "bf16":
        y = ss2d_inputs.round_to_bf16(y)
    g = rng.uniform(0.5, 1.5, D).astype(np.float32)
    b = rng.standard_normal(D).astype(np.float32) * 0.1
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = _lib().channel_last(torch.from_numpy(y).to(tdt).cuda(), torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    ref = oepi.layer_norm_channel_last(y, g, b, eps=1e-5)
    extra = 2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 0.0
    assert np.all(np.abs(out.double().cpu().numpy() - ref) <= 1e-5 * (1 + np.abs(ref)) + extra)


@pytest.mark.parametrize("shape", _shapes(404, 14), ids=lambda s: "x".join(map(str, s)))
def test_backward_random(shape):
    B, D, H, W, N, dtype = shape
    print(f"[random backward] {shape}", flush=True)
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=B * 3 + D + H + W + N, dtype=dtype)
    dy = np.random.default_rng(D + N).standard_normal((B, D, H, W)).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        dy = ss2d_inputs.round_to_bf16(dy)
    d = {k: (torch.from_numpy(v).to(tdt) if k in ("x", "dt", "Bs", "Cs") else torch.from_numpy(v)).cuda()
         for k, v in inp.items()}
    got = _lib().backward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"],
                          torch.from_numpy(dy).to(tdt).cuda())
    torch.cuda.synchronize()
    ref = obwd.ss2d_backward_f64(**inp, dy=dy)
    io = 1e-2 if dtype == "bf16" else 1e-5  # bf16 outputs carry their rounding
    tol = {"dx": io, "ddt": io, "dBs": io, "dCs": io, "dA_log": 1e-4, "ddt_bias": 1e-4, "dDs": 1e-4}
    for k, r in ref.items():
        g = got[k].double().cpu().numpy()
        rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
        assert rel <= tol[k], (k, rel)
