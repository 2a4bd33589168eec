"""The C ABI driven from C on the GPU: tests/c_abi_gpu.c (HIP runtime API and
include/sage_attn.h only, no Python or torch in that process) runs prep and
forward on seeded inputs written here.  Its output must equal the Python
binding's bit for bit (same kernels, same launches) and meet the parity bars
against the oracle on every row."""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import sage_oracle as so
from quantized_exact_attention_amd import build as qbuild
from quantized_exact_attention_amd import sage
from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs
from tests import test_gpu_parity as tp

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def binary(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    out = tmp_path_factory.mktemp("cabi_gpu") / "c_abi_gpu"
    libdir = os.path.dirname(qbuild.LIB_PATH)
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "c_abi_gpu.c"),
           "-L", libdir, "-lsage_attn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + libdir, "-o", str(out)]
    subprocess.run(cmd, check=True)
    return str(out)


@pytest.mark.parametrize("D,single_pass", [(128, False), (64, True)])
def test_c_caller_matches_binding_and_oracle(binary, tmp_path, D, single_pass):
    B, H, Nq, Nkv = 1, 3, 300, 500
    q, k, v = make_inputs(WORKLOADS["ragged_tails"], seed=40 + D, B=B, H=H, Nq=Nq, Nkv=Nkv, D=D)
    paths = {n: str(tmp_path / (n + ".bin")) for n in "qkvo"}
    for n, t in zip("qkv", (q, k, v)):
        t.contiguous().view(torch.int16).numpy().tofile(paths[n])
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(
        p for p in (os.path.dirname(qbuild.LIB_PATH), os.path.join(ROCM, "lib"), env.get("LD_LIBRARY_PATH")) if p)
    print("  C caller B=%d H=%d Nq=%d Nkv=%d D=%d single_pass=%s" % (B, H, Nq, Nkv, D, single_pass), flush=True)
    res = subprocess.run([binary, str(B), str(H), str(Nq), str(Nkv), str(D), paths["q"], paths["k"], paths["v"],
                          paths["o"], str(int(single_pass))], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stderr
    o_c = np.fromfile(paths["o"], dtype=np.uint16).reshape(B, H, Nq, D)

    dev = torch.device("cuda:0")
    quant = sage.sage_quant_prep(q.to(dev), k.to(dev), v.to(dev), single_pass=single_pass)
    o_py = sage.sage_attn_fwd(quant).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(o_c, o_py)

    stats = tp.OStats()
    for h in range(H):
        _, O_ref = so.attention_bh(q[0, h].float().numpy(), k[0, h].float().numpy(), v[0, h].float().numpy())
        stats.add_o(o_c[0, h], O_ref)
    stats.check()
