"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sage_attn.h, sizes buffers, and rejects bad arguments with
the documented status before any HIP call."""

import ctypes
import os
import re

import pytest

from quantized_exact_attention_amd import build as qbuild
from quantized_exact_attention_amd import sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qbuild.LIB_PATH):
        qbuild.build()
    return sage.lib()


@pytest.fixture(scope="module")
def no_gfx950(L):
    """For tests whose calls pass validation with made-up device addresses:
    they rely on the library stopping at its device check, so they must not run
    where a gfx950 GPU would take the launch."""
    if L.sage_device_check(0) == 0:
        pytest.skip("a gfx950 device is present: made-up device addresses would reach a kernel")


def header_functions():
    text = open(os.path.join(ROOT, "include", "sage_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_\w+)\s*\(", text)))


def test_exports_every_header_function(L):
    names = header_functions()
    assert {"sage_quant_prep", "sage_quant_prep_single_pass", "sage_attn_fwd", "sage_attn_fwd_capture",
            "sage_buffer_bytes", "sage_status_string", "sage_device_check"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for st in range(-9, 1):
        assert sage.status_string(st) not in ("", "unknown status")
    assert sage.status_string(-99) == "unknown status"


def test_buffer_bytes_formulas(L):
    B, H, Nq, Nkv, D = 2, 3, 1000, 333, 128
    nqb, T = 8, 6
    expect = [B * H * nqb * 128 * D, B * H * nqb * 4, B * H * T * 64 * D, B * H * T * 4,
              B * H * T * 64 * D, B * H * D * 4, B * H * D * 4]
    for which, e in enumerate(expect):
        assert sage.sage_buffer_bytes(B, H, Nq, Nkv, D, which) == e
    assert sage.sage_buffer_bytes(B, H, Nq, Nkv, D, 7) > 0


@pytest.mark.parametrize("shape,status", [
    ((1, 1, 128, 64, 96), -3), ((1, 1, 0, 64, 64), -2), ((1, 1, 64, 0, 64), -2),
    ((0, 1, 64, 64, 64), -2), ((300, 300, 64, 64, 64), -2), ((1, 65536, 8, 8, 64), -2),
    ((2, 32768, 8, 8, 64), -2), ((1, 1, (1 << 28) + 1, 64, 64), -2), ((1, 1, 64, (1 << 28) + 1, 64), -2)])
def test_buffer_bytes_rejects_bad_shapes(L, shape, status):
    n = ctypes.c_size_t()
    s = sage.SageShape(*shape)
    assert L.sage_buffer_bytes(ctypes.byref(s), 0, ctypes.byref(n)) == status
    assert L.sage_buffer_bytes(None, 0, ctypes.byref(n)) == -1
    assert L.sage_buffer_bytes(ctypes.byref(sage.SageShape(1, 1, 8, 8, 64)), 9, ctypes.byref(n)) == -8


@pytest.mark.parametrize("shape", [(3, 21845, 8, 8, 64), (1, 65535, 1, 1, 128), (1, 1, 1 << 28, 1 << 28, 128)])
def test_buffer_bytes_accepts_the_limits(L, shape):
    """B*H = 65535 (the prep's second grid dimension) and Nq = Nkv = 2^28 are accepted."""
    n = ctypes.c_size_t()
    assert L.sage_buffer_bytes(ctypes.byref(sage.SageShape(*shape)), 0, ctypes.byref(n)) == 0
    B, H, Nq, _, D = shape
    assert n.value == B * H * (-(-Nq // 128)) * 128 * D


def _fake_quant(base=1 << 40, step=1 << 30):
    q = sage.SageQuantC(*[base + i * step for i in range(8)])
    return q


def _strides(B, H, N, D):
    st = sage.SageStrides()
    for f in ("q", "k", "v", "o"):
        getattr(st, f)[:] = [H * N * D, N * D, D]
    return st


@pytest.mark.parametrize("entry", ["sage_quant_prep", "sage_quant_prep_single_pass"])
def test_prep_validation_before_any_hip_call(L, entry):
    shape = sage.SageShape(1, 2, 100, 100, 64)
    st = _strides(1, 2, 100, 64)
    qc = _fake_quant()
    q, k, v = 1 << 36, 2 << 36, 3 << 36
    call = lambda *a: getattr(L, entry)(*a)
    assert call(q, k, v, None, ctypes.byref(st), ctypes.byref(qc), None) == -1
    assert call(None, k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), None) == -1
    assert call(q, k, v, ctypes.byref(shape), ctypes.byref(st), None, None) == -1
    assert call(q + 2, k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), None) == -4
    bad = _strides(1, 2, 100, 64)
    bad.k[2] = 68
    assert call(q, k, v, ctypes.byref(shape), ctypes.byref(bad), ctypes.byref(qc), None) == -4
    alias = _fake_quant(base=q)  # q_codes starts where q does
    assert call(q, k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(alias), None) == -5
    d96 = sage.SageShape(1, 2, 100, 100, 96)
    assert call(q, k, v, ctypes.byref(d96), ctypes.byref(st), ctypes.byref(qc), None) == -3


@pytest.mark.parametrize("entry", ["sage_attn_fwd", "sage_attn_fwd_paired"])
def test_fwd_validation_before_any_hip_call(L, entry, no_gfx950):
    shape = sage.SageShape(2, 2, 300, 77, 128)
    st = _strides(2, 2, 300, 128)
    qc = _fake_quant()
    out = 1 << 36
    f = getattr(L, entry)
    assert f(None, ctypes.byref(shape), 0.0, out, ctypes.byref(st), None) == -1
    assert f(ctypes.byref(qc), ctypes.byref(shape), 0.0, None, ctypes.byref(st), None) == -1
    assert f(ctypes.byref(qc), ctypes.byref(shape), 0.0, out + 8, ctypes.byref(st), None) == -4
    assert f(ctypes.byref(qc), ctypes.byref(shape), float("nan"), out, ctypes.byref(st), None) == -8
    # output overlapping the K codes buffer
    assert f(ctypes.byref(qc), ctypes.byref(shape), 0.0, qc.k_codes + 4096, ctypes.byref(st), None) == -5
    # output strides under which two elements share an address
    for o in ([300 * 128, 300 * 128, 128], [2 * 300 * 128, 300 * 128, 0], [0, 300 * 128, 128],
              [256, 128, 384], [2 * 300 * 128, 64, 256]):
        self_overlap = _strides(2, 2, 300, 128)
        self_overlap.o[:] = o
        assert f(ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(self_overlap), None) == -5, o
    # valid layouts get past the check (then fail on the missing device, not on aliasing)
    for o in ([300 * 128 * 2, 128, 256], [256, 128, 512], [2 * 300 * 136, 300 * 136, 136]):
        ok = _strides(2, 2, 300, 128)
        ok.o[:] = o
        assert f(ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(ok), None) not in (-4, -5), o
    nulls = _fake_quant()
    nulls.v_scale = None
    assert f(ctypes.byref(nulls), ctypes.byref(shape), 0.0, out, ctypes.byref(st), None) == -1
    # the forward does not read the workspace, so a NULL one passes validation
    no_ws = _fake_quant()
    no_ws.workspace = None
    assert f(ctypes.byref(no_ws), ctypes.byref(shape), 0.0, out, ctypes.byref(st), None) in (0, -6, -7)
    cap = L.sage_attn_fwd_capture
    caps = [1 << 37, 1 << 38, 1 << 39, 1 << 40, 1 << 41, 1 << 42]
    assert cap(ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(st), None, 1, *caps, None) == -1
    assert cap(ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(st), 1 << 35, 0, *caps, None) == -8
    for i in range(3, 6):                       # partial, RO and reciprocal buffers are required too
        missing = list(caps)
        missing[i] = None
        assert cap(ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(st), 1 << 35, 1,
                   *missing, None) == -1
    misaligned = list(caps)
    misaligned[4] += 4
    assert cap(ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(st), 1 << 35, 1,
               *misaligned, None) == -4


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(sage, "_lib", None)
    monkeypatch.setattr(sage, "LIB_PATH", "/nonexistent/libsage_attn.so")
    with pytest.raises(RuntimeError):
        sage.lib()


def test_no_alloc_prep_rejects_shapes_beyond_its_scratch(L, no_gfx950):
    """The allocation-free prep checks its static 8 MiB scratch against the
    shape before any HIP call; a NULL workspace is accepted there."""
    f = L.sage_quant_prep_no_alloc
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.POINTER(sage.SageShape), ctypes.POINTER(sage.SageStrides),
                                          ctypes.POINTER(sage.SageQuantC), ctypes.c_void_p]
    f.restype = ctypes.c_int
    big = sage.SageShape(1, 64, 128, 65536, 128)
    assert sage.sage_buffer_bytes(1, 64, 128, 65536, 128, 7) > 8 << 20
    qc = _fake_quant()
    qc.workspace = None
    st = _strides(1, 64, 128, 128)
    st.k[:] = st.v[:] = [64 * 65536 * 128, 65536 * 128, 128]
    base = 1 << 44
    assert f(base, base + (1 << 40), base + (1 << 41), ctypes.byref(big), ctypes.byref(st), ctypes.byref(qc),
             None) == -9
    # within the scratch the same call passes validation and stops at the device check (no GPU here)
    small = sage.SageShape(1, 2, 128, 1000, 128)
    st = _strides(1, 2, 128, 128)
    st.k[:] = st.v[:] = [2 * 1000 * 128, 1000 * 128, 128]
    r = f(base, base + (1 << 40), base + (1 << 41), ctypes.byref(small), ctypes.byref(st), ctypes.byref(qc), None)
    assert r in (0, -6, -7)
    nulls = _fake_quant()
    nulls.k_codes = None
    assert f(base, base + (1 << 40), base + (1 << 41), ctypes.byref(small), ctypes.byref(st), ctypes.byref(nulls),
             None) == -1


def test_race_gate_validation_before_any_hip_call(L, no_gfx950):
    f = L.sage_race_gate
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.POINTER(sage.SageShape), ctypes.POINTER(sage.SageStrides),
                                          ctypes.POINTER(sage.SageQuantC), ctypes.c_float, ctypes.c_void_p,
                                          ctypes.c_uint32, ctypes.c_void_p]
    f.restype = ctypes.c_int
    shape = sage.SageShape(1, 2, 100, 100, 64)
    st = _strides(1, 2, 100, 64)
    qc = _fake_quant()
    q, k, v, out = 1 << 44, (1 << 44) + (1 << 36), (1 << 44) + (2 << 36), (1 << 44) + (3 << 36)
    assert f(q, k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), 0.0, out, 0, None) == -8
    assert f(q, k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), 0.0, q, 5, None) == -5
    assert f(q, k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), 0.0, None, 5, None) == -1
    assert f(q, k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), 0.0, out, 5, None) in (-6, -7, 0)


def test_mfma_peak_sample_validation_before_any_hip_call(L, no_gfx950):
    f = L.sage_mfma_peak_sample
    dst = 1 << 44
    assert f(0, 16, None, None) == -1
    assert f(0, 16, dst + 2, None) == -4
    for kind, iters in ((2, 16), (-1, 16), (0, 0), (1, -5), (1, 65537)):
        assert f(kind, iters, dst, None) == -8, (kind, iters)
    assert f(1, 65536, dst, None) in (0, -6, -7)


def test_valu_sample_validation_before_any_hip_call(L, no_gfx950):
    f = L.sage_valu_sample
    dst = 1 << 44
    assert f(0, 16, None, None) == -1
    assert f(0, 16, dst + 2, None) == -4
    for mix, kc in ((6, 16), (-1, 16), (0, 0), (5, -5), (1, 10001)):
        assert f(mix, kc, dst, None) == -8, (mix, kc)
    assert f(5, 10000, dst, None) in (0, -6, -7)


def test_kv_prep_validation_before_any_hip_call(L, no_gfx950):
    """The K/V-only prep takes no q and accepts NULL Q codes and scale."""
    f = L.sage_quant_prep_kv
    shape = sage.SageShape(1, 2, 1, 100, 64)
    st = _strides(1, 2, 100, 64)
    qc = _fake_quant()
    qc.q_codes = None
    qc.q_scale = None
    k, v = 2 << 36, 3 << 36
    assert f(None, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), None) == -1
    assert f(k, v, ctypes.byref(shape), None, ctypes.byref(qc), None) == -1
    assert f(k + 4, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), None) == -4
    nokm = _fake_quant()
    nokm.q_codes = None
    nokm.k_mean = None
    assert f(k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(nokm), None) == -1
    alias = _fake_quant(base=k)                  # q_codes (ignored) at k; k_codes right after it
    alias.q_codes = None
    alias.k_codes = k
    assert f(k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(alias), None) == -5
    assert f(k, v, ctypes.byref(shape), ctypes.byref(st), ctypes.byref(qc), None) in (0, -6, -7)


def test_q_quantizing_fwd_validation_before_any_hip_call(L, no_gfx950):
    f = L.sage_attn_fwd_q
    shape = sage.SageShape(2, 2, 300, 128, 128)
    st = _strides(2, 2, 300, 128)
    qc = _fake_quant()
    qc.q_codes = None
    qc.q_scale = None
    qc.workspace = None
    q, out = 1 << 45, (1 << 45) + (1 << 36)
    assert f(None, ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(st), None) == -1
    assert f(q, ctypes.byref(qc), ctypes.byref(shape), 0.0, None, ctypes.byref(st), None) == -1
    assert f(q + 8, ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(st), None) == -4
    bad = _strides(2, 2, 300, 128)
    bad.q[2] = 132
    assert f(q, ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(bad), None) == -4
    assert f(q, ctypes.byref(qc), ctypes.byref(shape), 0.0, q + 256, ctypes.byref(st), None) == -5
    assert f(q, ctypes.byref(qc), ctypes.byref(shape), float("nan"), out, ctypes.byref(st), None) == -8
    assert f(q, ctypes.byref(qc), ctypes.byref(shape), 0.0, out, ctypes.byref(st), None) in (0, -6, -7)
