"""GPU parity of the backward (ss2d_backward) against the float64 backward oracle
(oracle/backward.py), gradient by gradient, through the C ABI.

Tolerances (fp32 arithmetic, u = 2^-24 ~ 6e-8).  Per-element gradients (dx, ddt,
dBs, dCs) are sums of at most 4N or D products after recurrences whose decays are
below 1, so rounding stays near sqrt(n) u relative: relative L2 <= 1e-5, as for
the forward.  The per-channel parameter gradients (dA_log, ddt_bias, dDs) are sums
over the batch and every step, up to ~10^5 terms with cancellation:
relative L2 <= 1e-4.
"""
import numpy as np
import pytest

from oracle import backward
import ss2d_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = {"dx": 1e-5, "ddt": 1e-5, "dBs": 1e-5, "dCs": 1e-5, "dA_log": 1e-4, "ddt_bias": 1e-4, "dDs": 1e-4}


def _run(B, D, H, W, N, seed, a_log="random"):
    inp = ss2d_inputs.tiny_random(B, D, H, W, N, seed=seed, a_log=a_log)
    rng = np.random.default_rng(seed + 7)
    dy = rng.standard_normal((B, D, H, W)).astype(np.float32)
    d = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    import selective_scan_crossscan_amd as ss2d
    got = ss2d.backward(d["x"], d["dt"], d["A_log"], d["dt_bias"], d["Bs"], d["Cs"], d["Ds"],
                        torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    ref = backward.ss2d_backward_f64(**inp, dy=dy)
    errs = {}
    for k, r in ref.items():
        g = got[k].double().cpu().numpy()
        assert g.shape == r.shape, k
        errs[k] = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= TOL[k], (k, e)
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
