"""The two measurement entry points of the C ABI on the GPU: the per-unit
shader-clock sample and the matrix-core peak sample that bench.py reports
beside the nominal peak."""

import pytest
import torch

import bench
from quantized_exact_attention_amd import sage

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_clock_sample_gives_a_plausible_clock_on_most_units():
    """Two samples around busy matrix work on every SIMD (an idle unit may be
    clock-gated, and its counter then barely moves)."""
    clk = torch.zeros(2, sage.CLOCK_SAMPLES, 4, dtype=torch.int64, device=DEV)
    dst = torch.zeros(sage.PEAK_WORKGROUPS * 256, dtype=torch.int32, device=DEV)
    sage.sage_mfma_peak_sample(0, 1, dst)
    sage.sage_clock_sample(clk[0])
    torch.cuda.synchronize()
    sage.sage_clock_sample(clk[0])
    sage.sage_mfma_peak_sample(0, 4096, dst)
    sage.sage_clock_sample(clk[1])
    torch.cuda.synchronize()
    s = bench.shader_clock_ghz(clk.cpu().numpy())
    assert s is not None
    print("  clock over a matrix-instruction stream: median %.3f GHz (%.3f-%.3f), %d units"
          % (s["median"], s["min"], s["max"], s["units"]), flush=True)
    assert s["units"] >= 200                      # 256 compute units; 2048 workgroups reach nearly all
    assert 0.5 < s["min"] <= s["median"] <= s["max"] < 3.0


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_peak_sample_runs_near_the_matrix_peak(kind):
    dst = torch.zeros(sage.PEAK_WORKGROUPS * 256, dtype=torch.int32, device=DEV)
    sage.sage_mfma_peak_sample(kind, 1, dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    ops = sage.sage_mfma_peak_sample(kind, 2048, dst)
    b.record()
    torch.cuda.synchronize()
    rate = ops / (a.elapsed_time(b) * 1e-3) / 1e12
    print("  %s matrix instruction stream: %.0f TOP/s" % ("INT8 32x32x32" if kind == 0 else "FP8 32x32x64", rate),
          flush=True)
    assert torch.count_nonzero(dst).item() > 0
    # 5.0 P ops/s nominal at 2.4 GHz; the clock under this load is lower, and
    # half the nominal rate would mean the stream is not feeding every SIMD
    assert 2500 < rate < 5200
    with pytest.raises(sage.SageError):
        sage.sage_mfma_peak_sample(2, 16, dst)


def test_valu_sample_rates_are_ordered_as_the_issue_model_says():
    """More issuing waves retire more FMAs per cycle; exp costs more than FMA;
    a matrix-instruction stream on the same SIMD slows the vector work."""
    dst = torch.zeros(3 * 16 * sage.VALU_WORKGROUPS, dtype=torch.int32, device=DEV)
    rates = {}
    for mix in range(len(sage.VALU_MIXES)):
        sage.sage_valu_sample(mix, 100, dst)
        torch.cuda.synchronize()
        words = dst.view(sage.VALU_WORKGROUPS, 16, 3).cpu().numpy()
        roles = sage.VALU_MIXES[mix]
        for g, role in enumerate(roles):          # idle waves report 0 rounds, active ones at least one
            rounds = words[:, 4 * g:4 * g + 4, 0]
            assert (rounds == 0).all() if role == 0 else (rounds >= 1).all(), (mix, g)
        rates[mix] = bench.valu_rates(words, mix)
        print("  mix %d %s: %s" % (mix, roles, {k: round(v, 2) for k, v in rates[mix].items()}), flush=True)
    fma1, fma3, fma4, exp3 = rates[0]["fma"], rates[1]["fma"], rates[2]["fma"], rates[3]["exp"]
    assert 1.0 < fma4 <= fma3 * 1.05 and fma3 < fma1 < 20.0
    assert fma3 < exp3 < 30.0
    assert rates[4]["fma"] > fma3 and rates[5]["exp"] > exp3
    assert 20.0 < rates[4]["matrix"] < 80.0
    with pytest.raises(sage.SageError):
        sage.sage_valu_sample(len(sage.VALU_MIXES), 10, dst)
