"""Build the gfx950 HIP library in-tree: quantized_exact_attention_amd/lib/libsage_attn.so.

Every source is compiled for gfx950 only, with FP contraction off (the kernels
call fma explicitly where they want one), packed-FP32 instruction selection
disabled and matrix-instruction results kept in VGPRs.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libsage_attn.so")
SOURCES = ["sage_prep.hip", "sage_fwd.hip", "sage_abi.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-instruction accumulators in VGPRs: the softmax and the RO update
    # read them directly instead of copying every value out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile all HIP sources (in parallel) and link the shared library."""
    os.makedirs(LIB_DIR, exist_ok=True)
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="sage_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            cmd = [cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        for cmd, pr in procs:
            out, _ = pr.communicate()
            text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                             if "not a recognized feature" not in l)
            if pr.returncode != 0:
                raise RuntimeError("hipcc failed: %s\n%s" % (" ".join(cmd), text))
            if verbose and text.strip():
                print(text)
        tmp_lib = LIB_PATH + ".tmp"
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if res.returncode != 0:
            raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), res.stdout.decode(errors="replace")))
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
