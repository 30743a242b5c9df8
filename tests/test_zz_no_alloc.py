"""The no-allocation forward (ss2d_forward_noalloc) against ss2d_forward and the fp64
oracle, through the C ABI.  It runs from one static device array, so two calls in a
row (the second smaller) must both be right, and each must equal what ss2d_forward
computes on the same inputs to the forward's tolerances (fp32: rel-L2 <= 1e-5 and
max |err| <= 1e-4 max|y|; bf16: rel-L2 <= 2e-2)."""
import numpy as np
import pytest

import oracle
import ss2d_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    import selective_scan_crossscan_amd as ss2d
    return ss2d


def _dev(inp, dtype):
    t = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(t if k in ("x", "dt", "Bs", "Cs") else torch.float32)
            .cuda() for k, v in inp.items()}


def _check(y, ref, dtype, label):
    d = y - ref
    rel = float(np.linalg.norm(d) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(d)))
    print(f"[noalloc] {label}: rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    if dtype == "bf16":
        assert rel <= 2e-2, (label, rel)
    else:
        assert rel <= 1e-5 and mx <= 1e-4 * float(np.max(np.abs(ref))), (label, rel, mx)


def _run_both(shape, dtype, seed):
    B, D, H, W, N = shape
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=seed, dtype=dtype)
    d = _dev(inp, dtype)
    code = 1 if dtype == "bf16" else 0
    y_na = torch.full((B, D, H, W), float("nan"), dtype=d["x"].dtype, device="cuda")
    y_ref = torch.empty_like(y_na)
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [d[k].data_ptr() for k in ("x", "dt", "A_log", "dt_bias", "Bs", "Cs", "Ds")]
    print(f"[case] noalloc {shape} {dtype}", flush=True)
    rc = _lib().ss2d_forward_noalloc(*ptrs, y_na.data_ptr(), B, D, H, W, N, code, stream)
    assert rc == 0, _lib().status_string(rc)
    rc = _lib().ss2d_forward(*ptrs, y_ref.data_ptr(), B, D, H, W, N, code, stream)
    assert rc == 0, _lib().status_string(rc)
    torch.cuda.synchronize()
    a = y_na.double().cpu().numpy()
    b = y_ref.double().cpu().numpy()
    assert np.all(np.isfinite(a))
    _check(a, b, dtype, f"{shape} {dtype} vs ss2d_forward")
    return inp, a


PAIRS = [
    # (first call, second smaller call), dtype
    (((2, 64, 56, 56, 16), (1, 16, 9, 14, 16)), "f32"),      # transposing plan vs in-place gathers
    (((1, 5, 72, 72, 16), (1, 3, 40, 40, 7)), "f32"),        # segmented, then a fused plan
    (((2, 9, 28, 28, 40), (1, 4, 10, 20, 16)), "bf16"),      # bf16: row and column planes in the array
]


@pytest.mark.parametrize("pair,dtype", PAIRS)
def test_noalloc_two_calls_match_forward(pair, dtype):
    for i, shape in enumerate(pair):
        inp, y = _run_both(shape, dtype, seed=100 + i)
        if np.prod(shape) <= 2e6:
            _check(y, oracle.ss2d_inputs_f64(inp), dtype, f"{shape} {dtype} vs oracle")


def test_noalloc_stage1_full_size():
    """VMamba-T stage-1 (fp32, 77 MB of temporary) from the static array."""
    shape = ss2d_inputs.CONFIGS[1]
    _run_both((shape.B, shape.D, shape.H, shape.W, shape.N), "f32", seed=0)


def test_noalloc_limit_is_refused():
    # distinct fake addresses: refused on the plan's size before any device work
    ptrs = [(1 << 40) + i * (1 << 34) for i in range(8)]
    rc = _lib().ss2d_forward_noalloc(*ptrs, 64, 384, 28, 28, 16, 1, None)
    assert rc == -9
