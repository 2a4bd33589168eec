"""bench.py's host-side logic, no GPU: the one-GPU refusal and the clock
computation from two counter samples."""

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
