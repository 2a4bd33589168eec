"""bench.py's host-side logic, no GPU: the one-GPU refusal, the clock
computation from two counter samples and the vector-issue rates."""

import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_shader_clock_from_two_samples():
    """Units are matched by (XCD, hardware-id bits 8-14); the clock of a unit is
    its counter delta over the 100 MHz counter delta."""
    n = 16
    a = np.zeros((n, 4), np.int64)
    b = np.zeros((n, 4), np.int64)
    for i in range(n):
        xcd, cu = i % 8, i // 8
        hwid = (cu << 8) | 0x33                   # low bits (wave, SIMD) must not matter
        a[i] = (1000, 500, xcd, hwid)
        ghz = 2.0 + 0.01 * i
        b[i] = (1000 + int(ghz * 10 * 1000), 500 + 1000, xcd, hwid ^ 0x3)   # 1000 ticks of 100 MHz = 10 us
    s = bench.shader_clock_ghz(np.stack([a, b]))
    assert s["units"] == n
    assert abs(s["min"] - 2.0) < 1e-9 and abs(s["max"] - 2.15) < 1e-9
    assert abs(s["median"] - np.median([2.0 + 0.01 * i for i in range(n)])) < 1e-9


def test_valu_rates_sum_the_waves_of_a_role_per_simd():
    """Per SIMD, a role's instructions per cycle are the sum over its waves;
    the cycles per instruction reported is the median over SIMDs."""
    from quantized_exact_attention_amd import sage
    mix = 4                                       # {matrix, FMA, FMA, FMA}
    words = np.zeros((sage.VALU_WORKGROUPS, 16, 3), np.int64)
    for g in range(sage.VALU_WORKGROUPS):
        for w in range(16):
            role = sage.VALU_MIXES[mix][w // 4]
            words[g, w, 1] = 100000               # cycles
            # each FMA wave retires one instruction per 15 cycles: 3 waves -> 5 cycles each
            words[g, w, 0] = 100000 // (15 * 64) if role == 1 else 100000 // (40 * 16)
    r = bench.valu_rates(words, mix)
    assert abs(r["fma"] - 100000 / (3 * (100000 // (15 * 64)) * 64)) < 1e-9
    assert abs(r["matrix"] - 100000 / ((100000 // (40 * 16)) * 16)) < 1e-9
    assert bench.valu_rates(words, 0).keys() == {"fma"}
