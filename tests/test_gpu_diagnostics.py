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
