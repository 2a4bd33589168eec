"""bench.py's one JSON line on the GPU: the keys the benchmark contract names,
with the roofline and CPU-oracle objects, on the single-tile workload (a few
seconds)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract_keys():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "single_tile", "--steps", "5",
                        "--warmup", "5", "--cpu-budget", "1", "--cpu-workers", "2"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 5 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["config"]["workload"] == "single_tile"
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 5000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-12
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["unit"] == "TFLOPS"
    for key in ("fwd_single_launch", "fwd_back_to_back", "mfma_peak_measured", "valu_rates_measured",
                "sustained_sclk_ghz", "q_quantizing_pair"):
        assert key in d, key
    assert d["q_quantizing_pair"]["output_equal"] is True
