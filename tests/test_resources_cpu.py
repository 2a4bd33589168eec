"""Resource gate on the build, no GPU needed: the compiler's resource report
for every kernel of the library.  The pages' prototype was gated on zero
spills and zero local memory ("Experiment Log", Phase 2A VEA-B Capability
Decision and Phase 2B); here every kernel runs without scratch except the
forward's capture build, which only the tests launch, and the default forward
keeps the occupancy its schedule is built for (three waves per SIMD at
D = 128, five at D = 64)."""

import os
import re
import subprocess
import tempfile

import pytest

from quantized_exact_attention_amd import build as qbuild

SOURCES = ["sage_prep.hip", "sage_fwd.hip", "sage_abi.hip"]


def _report(src):
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [qbuild.hipcc(), *qbuild.HIPCC_FLAGS, "--cuda-device-only", "-c", os.path.join(qbuild.CSRC, src),
               "-o", os.path.join(tmp, "x.o"), "-Rpass-analysis=kernel-resource-usage"]
        out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, check=True).stdout.decode()
    kernels, cur = {}, None
    for line in out.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                      r"LDS Size \[bytes/block\]): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).split(" ")[0]] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def report():
    rep = {}
    for src in SOURCES:
        rep.update(_report(src))
    return rep


def _fwd(report, D, capture, race, qpw, qin=0):
    name = "_ZN4sage10k_attn_fwdILi%dELb%dELb%dELi%dELb%dEEEvNS_9FwdParamsE" % (D, capture, race, qpw, qin)
    assert name in report, sorted(report)
    return report[name]


def test_every_kernel_but_the_capture_build_runs_without_scratch(report):
    assert len(report) >= 20
    for name, r in report.items():
        if "k_attn_fwd" in name and "Lb1ELb0ELi1ELb0E" in name:      # capture build: tests only
            continue
        assert r["ScratchSize"] == 0, (name, r)


@pytest.mark.parametrize("D,waves", [(128, 3), (64, 5)])
def test_default_forward_keeps_its_occupancy(report, D, waves):
    r = _fwd(report, D, 0, 0, 1)
    assert r["Occupancy"] == waves and r["ScratchSize"] == 0, r
    assert r["LDS"] == 2 * 2 * 64 * D                       # two [K tile | V tile] buffers


def test_race_gate_paired_and_q_quantizing_builds_match_the_default_occupancy(report):
    for D, waves in ((128, 3), (64, 5)):
        for capture, race, qpw, qin in ((0, 1, 1, 0), (0, 0, 3, 0), (0, 0, 1, 1)):
            r = _fwd(report, D, capture, race, qpw, qin)
            assert r["Occupancy"] == waves and r["ScratchSize"] == 0, r
