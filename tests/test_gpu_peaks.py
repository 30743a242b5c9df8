"""On-device roofline probes (ss2d_measure_peaks): the rates must be positive and
inside what a gfx950 part can physically reach, and keep their expected order
(a transcendental is slower than an FMA; the update mix is slower than either
alone; a copy moves no more bytes per second than HBM can read).

Upper bounds come from the vendor's unit counts at 2.4 GHz with headroom for a
faster clock: 256 CUs x 64 fp32 lanes/clk (non-packed FMA), half of that for
exp2 (CDNA4 doubled the transcendental rate of CDNA3), 8 TB/s HBM3E (plus a margin for lines the 256 MB MALL still holds), and
256 bytes/clk/CU of LDS.
"""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CLK = 2.6e9  # a little above the 2.4 GHz peak clock


def test_measured_peaks_are_physical():
    import selective_scan_crossscan_amd as ss2d
    p = ss2d.measure_peaks(1 << 30)
    print({k: f"{v:.4g}" for k, v in p.items()})
    ncu = p["compute_units"]
    assert ncu == torch.cuda.get_device_properties(0).multi_processor_count
    fma_max = ncu * 64 * CLK
    assert 0.2 * fma_max < p["fma_per_s"] <= fma_max, p
    assert 0.2 * fma_max / 2 < p["exp_per_s"] <= fma_max / 2 * 1.01, p
    assert p["update_mix_per_s"] < 1.02 * min(p["exp_per_s"], p["fma_per_s"]), p
    assert p["update_mix_per_s"] > 0.2 * fma_max / 8, p
    # the scan's state loop issues more than the update's minimum (fold and replay,
    # prefix combine), so it runs below the update mix, but not by 3x
    assert p["update_mix_per_s"] / 3 < p["state_loop_per_s"] < p["update_mix_per_s"], p
    assert 1e12 < p["hbm_read_Bps"] <= 1e13, p
    assert 1e12 < p["hbm_copy_Bps"] <= 1e13, p
    assert 0.1 * ncu * 128 * CLK < p["lds_read_Bps"] <= ncu * 256 * CLK, p


def test_measure_peaks_on_a_torch_stream():
    import selective_scan_crossscan_amd as ss2d
    s = torch.cuda.Stream()
    p = ss2d.measure_peaks(64 << 20, s.cuda_stream)
    assert all(v > 0 for v in p.values()), p
