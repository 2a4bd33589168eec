"""The allocation-free prep entry (sage_quant_prep_no_alloc, static device
scratch) called through the C ABI against sage_quant_prep (caller workspace):
every quantized buffer bit-identical, and the forward on either set gives the
same output bits.  Two calls in a row, the second on a smaller problem, so the
second runs on scratch the first left behind."""

import ctypes

import pytest
import torch

from quantized_exact_attention_amd import sage
from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

FIELDS = ("q_codes", "q_scale", "k_codes", "k_scale", "v_codes", "v_scale", "k_mean")


def _no_alloc_prep(qd, kd, vd, quant):
    """sage_quant_prep_no_alloc through the C ABI, with a NULL workspace."""
    st = sage.SageStrides()
    st.q, st.k, st.v = sage._strides3(qd), sage._strides3(kd), sage._strides3(vd)
    qc = quant.c_struct()
    qc.workspace = None
    stream = sage._stream_handle(None, qd.device)
    return sage.lib().sage_quant_prep_no_alloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                               ctypes.byref(quant.shape), ctypes.byref(st), ctypes.byref(qc),
                                               stream)


def _no_workspace_fwd(quant, out):
    """sage_attn_fwd through the C ABI with a NULL workspace (the forward does
    not use it)."""
    st = sage.SageStrides()
    st.o = sage._strides3(out)
    qc = quant.c_struct()
    qc.workspace = None
    return sage.lib().sage_attn_fwd(ctypes.byref(qc), ctypes.byref(quant.shape), ctypes.c_float(0.0),
                                    out.data_ptr(), ctypes.byref(st), sage._stream_handle(None, out.device))


def test_no_alloc_prep_matches_workspace_prep():
    dev = torch.device("cuda:0")
    lib = sage.lib()
    lib.sage_quant_prep_no_alloc.argtypes = [ctypes.c_void_p] * 3 + [
        ctypes.POINTER(sage.SageShape), ctypes.POINTER(sage.SageStrides), ctypes.POINTER(sage.SageQuantC),
        ctypes.c_void_p]
    lib.sage_quant_prep_no_alloc.restype = ctypes.c_int
    cases = [("dit_block", {}),                                           # 1.2 MiB of scratch
             ("ragged_tails", dict(B=1, H=3, Nq=300, Nkv=777, D=64))]     # then a smaller problem
    for name, over in cases:
        q, k, v = make_inputs(WORKLOADS[name], **over)
        print("  no-alloc prep:", name, tuple(q.shape), tuple(k.shape), flush=True)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        ref = sage.sage_quant_prep(qd, kd, vd)
        B, H, Nq, D = q.shape
        got = sage.SageQuant.allocate(B, H, Nq, k.shape[2], D, dev)
        for f in FIELDS:                       # stale contents must not matter
            getattr(got, f).view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats(dev).get("allocation.all.allocated", 0)
        assert _no_alloc_prep(qd, kd, vd, got) == 0
        assert torch.cuda.memory_stats(dev).get("allocation.all.allocated", 0) == before
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(ref, f).view(torch.uint8), getattr(got, f).view(torch.uint8)), (name, f)
        o_ref = sage.sage_attn_fwd(ref)
        o_got = torch.empty_like(o_ref)
        assert _no_workspace_fwd(got, o_got) == 0         # the whole path without any workspace
        torch.cuda.synchronize()
        assert torch.equal(o_ref.view(torch.int16), o_got.view(torch.int16)), name
        del ref, got, qd, kd, vd, o_ref, o_got
        torch.cuda.empty_cache()
