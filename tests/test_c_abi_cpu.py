"""The C ABI compiled against from C: tests/c_abi_check.c is built with the
host C compiler against include/sage_attn.h and the library, then run (no GPU
calls); its buffer sizes, struct sizes and status codes must equal the
binding's and the documented ones."""

import ctypes
import os
import shutil
import subprocess

import pytest

from quantized_exact_attention_amd import build as qbuild
from quantized_exact_attention_amd import sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    if not os.path.exists(qbuild.LIB_PATH):
        qbuild.build()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    out = tmp_path_factory.mktemp("cabi") / "c_abi_check"
    libdir = os.path.dirname(qbuild.LIB_PATH)
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir, "-lsage_attn",
           "-Wl,-rpath," + libdir, "-Wl,--allow-shlib-undefined", "-o", str(out)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(p for p in (libdir, "/opt/rocm/lib", env.get("LD_LIBRARY_PATH")) if p)
    text = subprocess.run([str(out)], check=True, capture_output=True, text=True, env=env).stdout
    return dict(line.split(" ", 1) for line in text.strip().splitlines())


def test_buffer_sizes_match_the_binding(results):
    shapes = [(2, 3, 300, 700, 128), (1, 1, 1, 1, 64), (3, 21845, 33, 70, 64)]
    for i, shape in enumerate(shapes):
        for w in range(8):
            status, n = results["buf_%d_%d" % (i, w)].split()
            assert int(status) == 0
            assert int(n) == sage.sage_buffer_bytes(*shape, w), (shape, w)


def test_status_word_offset(results):
    """The single pass's status word: after the K partials, the V partials and
    the V inverses (each region 256-byte aligned), behind BH arrival counters
    and BH ready flags, inside the workspace."""
    a256 = lambda x: (x + 255) // 256 * 256
    shapes = [(2, 3, 300, 700, 128), (1, 1, 1, 1, 64), (3, 21845, 33, 70, 64)]
    for i, (B, H, Nq, Nkv, D) in enumerate(shapes):
        status, off = (int(x) for x in results["status_off_%d" % i].split())
        BH, nchunk = B * H, -(-Nkv // 256)
        assert status == 0
        assert off == a256(BH * nchunk * D * 8) + a256(BH * nchunk * D * 4) + a256(BH * D * 4) + 8 * BH
        assert off % 4 == 0 and off + 4 <= sage.sage_buffer_bytes(B, H, Nq, Nkv, D, 7)
    assert int(results["status_off_null"]) == -1


def test_struct_sizes_match_the_binding(results):
    assert int(results["sizeof_shape"]) == ctypes.sizeof(sage.SageShape) == 20
    assert int(results["sizeof_strides"]) == ctypes.sizeof(sage.SageStrides) == 96
    assert int(results["sizeof_quant"]) == ctypes.sizeof(sage.SageQuantC) == 64


def test_validation_status_codes(results):
    assert int(results["bytes_null_shape"]) == -1          # SAGE_E_NULL
    assert int(results["bytes_bad_which"]) == -8           # SAGE_E_ARG
    assert int(results["bytes_bad_headdim"]) == -3         # SAGE_E_HEADDIM
    assert int(results["bytes_too_many_heads"]) == -2      # SAGE_E_SHAPE
    assert int(results["prep_null_inputs"]) == -1
    assert int(results["prep1_null_inputs"]) == -1
    assert int(results["prep_bad_shape"]) == -2
    assert int(results["fwd_null_out"]) == -1
    assert results["status_alias"] == sage.status_string(-5)
    assert results["status_unknown"] == "unknown status"
