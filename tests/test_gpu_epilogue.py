"""GPU parity of the channel-last epilogue (ss2d_channel_last) against the
float64 oracle in oracle/epilogue.py, element by element.

Tolerances.  The transpose alone is exact (bit-equal for both storage types).
The LayerNorm in fp32: the statistics are sums of D terms and the output is a
few operations on O(1) values, so |err| <= 1e-5 * (1 + |out|) elementwise (a
bound of the form D * 2^-24 * |terms| with D up to 1024 and margin).  bf16
storage adds the rounding of the output, 2^-8 |out|, and of the input, which the
oracle sees too (it reads the same bf16 values).
"""
import numpy as np
import pytest

from oracle import epilogue
import ss2d_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _lib():
    import selective_scan_crossscan_amd as ss2d
    return ss2d


def _case(B, D, H, W, dtype, seed):
    rng = np.random.default_rng(seed)
    # channels with their own offset and scale, so the statistics matter
    y = (rng.standard_normal((B, D, H, W)) * rng.uniform(0.5, 3.0, size=(1, D, 1, 1))
         + rng.standard_normal((1, D, 1, 1)) * 2.0).astype(np.float32)
    if dtype == "bf16":
        y = ss2d_inputs.round_to_bf16(y)
    g = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
    b = (rng.standard_normal(D) * 0.1).astype(np.float32)
    return y, g, b


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


# (B, D, H, W).  Channel-major fallback tiles (L or D not a multiple of the vector
# width, D above 900): 64 / 32 / 16 / 1 pixels per workgroup, ragged last tiles, odd
# D, the largest D.  Vector path (16-pixel pixel-major tiles): whole tiles, a 4- or
# 12-pixel last tile, 256- and 512-thread workgroups, bf16 with 8- and 4-element
# vectors, D at the vector path's limit (900) and just past it (904).
SHAPES = [(2, 16, 8, 8), (1, 192, 7, 9), (2, 384, 5, 7), (1, 768, 3, 5), (1, 3, 1, 37), (1, 4096, 2, 3),
          (3, 100, 6, 11),
          (2, 192, 8, 10), (1, 384, 6, 6), (2, 768, 4, 7), (1, 900, 4, 4), (1, 904, 2, 8), (3, 100, 4, 9),
          (1, 12, 2, 2), (4, 256, 16, 16), (2, 260, 4, 4)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_channel_last_norm_matches_oracle(shape, dtype):
    B, D, H, W = shape
    print(f"[epilogue] {shape} {dtype}", flush=True)
    y, g, b = _case(B, D, H, W, dtype, seed=D + H)
    ss2d = _lib()
    out = ss2d.channel_last(_dev(y, dtype), _dev(g), _dev(b), eps=1e-5)
    plain = ss2d.channel_last(_dev(y, dtype), normalize=False)
    torch.cuda.synchronize()
    ref = epilogue.layer_norm_channel_last(y, g, b, eps=1e-5)
    got = out.double().cpu().numpy()
    extra = 2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 0.0
    assert np.all(np.abs(got - ref) <= 1e-5 * (1 + np.abs(ref)) + extra)
    assert np.array_equal(plain.double().cpu().numpy(), epilogue.channel_last(y))


@pytest.mark.parametrize("D", [48, 384])  # gamma and beta in LDS, and read through the caches (wide rows)
def test_defaults_are_unit_scale_zero_shift(D):
    y, _, _ = _case(1, D, 4, 6, "f32", seed=3)
    out = _lib().channel_last(_dev(y))
    torch.cuda.synchronize()
    ref = epilogue.layer_norm_channel_last(y, eps=1e-5)
    assert np.all(np.abs(out.double().cpu().numpy() - ref) <= 1e-5 * (1 + np.abs(ref)))


def test_full_size_stage1_after_the_forward():
    # the forward's output at VMamba-T stage-1 size, then the epilogue
    shape = ss2d_inputs.CONFIGS[1]
    inp = ss2d_inputs.generate(shape, seed=0)
    d = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    ss2d = _lib()
    y = ss2d.forward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"])
    g = torch.linspace(0.5, 1.5, shape.D, device="cuda")
    b = torch.linspace(-0.1, 0.1, shape.D, device="cuda")
    out = ss2d.channel_last(y, g, b)
    torch.cuda.synchronize()
    ref = epilogue.layer_norm_channel_last(y.double().cpu().numpy(), g.cpu().numpy(), b.cpu().numpy(), eps=1e-5)
    assert np.all(np.abs(out.double().cpu().numpy() - ref) <= 1e-5 * (1 + np.abs(ref)))


def _offset(a, dtype):
    """A contiguous device tensor holding a whose base is one element past a 256-byte
    boundary (aligned to its element only)."""
    t = torch.bfloat16 if dtype == "bf16" else torch.float32
    flat = torch.zeros(a.size + 64, dtype=t, device="cuda")
    v = flat[1:1 + a.size].view(a.shape)
    v.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(t))
    return v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_element_aligned_bases_take_the_scalar_tiles(dtype):
    B, D, H, W = 2, 192, 8, 8
    y, g, b = _case(B, D, H, W, dtype, seed=9)
    ss2d = _lib()
    out = _offset(np.zeros((B, H, W, D), np.float32), dtype)
    ss2d.channel_last(_offset(y, dtype), _dev(g), _dev(b), eps=1e-5, out=out)
    torch.cuda.synchronize()
    ref = epilogue.layer_norm_channel_last(y, g, b, eps=1e-5)
    extra = 2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 0.0
    assert np.all(np.abs(out.double().cpu().numpy() - ref) <= 1e-5 * (1 + np.abs(ref)) + extra)


@pytest.mark.parametrize("ci", [1, 2, 3, 4])
def test_workload_shapes(ci):
    """The four workload shapes (the vector path) on random values, against the oracle on
    two batch elements."""
    shape = ss2d_inputs.CONFIGS[ci]
    B, D, H, W = 2, shape.D, shape.H, shape.W
    y, g, b = _case(B, D, H, W, shape.dtype, seed=ci)
    out = _lib().channel_last(_dev(y, shape.dtype), _dev(g), _dev(b), eps=1e-5)
    plain = _lib().channel_last(_dev(y, shape.dtype), normalize=False)
    torch.cuda.synchronize()
    ref = epilogue.layer_norm_channel_last(y, g, b, eps=1e-5)
    extra = 2.0 ** -8 * np.abs(ref) if shape.dtype == "bf16" else 0.0
    assert np.all(np.abs(out.double().cpu().numpy() - ref) <= 1e-5 * (1 + np.abs(ref)) + extra)
    assert np.array_equal(plain.double().cpu().numpy(), epilogue.channel_last(y))
