"""LDS race gate: the prep's three launches and the forward, built with
wave-uniform pseudo-random pauses before every LDS write and read and every
HBM -> LDS tile copy (sage_race_gate), must give the normal build's bits on
every quantized buffer and on the output.  The analogue of the race checks the
pages require ("Experiment Log", Phase 2A VEA-B Capability Decision: a
candidate with race hazards is rejected); here the check is that results do not
depend on the order in which waves reach shared memory."""

import ctypes

import pytest
import torch

from quantized_exact_attention_amd import sage
from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

FIELDS = ("q_codes", "q_scale", "k_codes", "k_scale", "v_codes", "v_scale", "k_mean")


def _race_gate(qd, kd, vd, quant, out, seed):
    L = sage.lib()
    f = L.sage_race_gate
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.POINTER(sage.SageShape), ctypes.POINTER(sage.SageStrides),
                                          ctypes.POINTER(sage.SageQuantC), ctypes.c_float, ctypes.c_void_p,
                                          ctypes.c_uint32, ctypes.c_void_p]
    f.restype = ctypes.c_int
    st = sage.SageStrides()
    st.q, st.k, st.v, st.o = (sage._strides3(t) for t in (qd, kd, vd, out))
    qc = quant.c_struct()
    return f(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), ctypes.byref(quant.shape), ctypes.byref(st),
             ctypes.byref(qc), 0.0, out.data_ptr(), seed, sage._stream_handle(None, qd.device))


@pytest.mark.parametrize("case", [("ragged_tails", {}),
                                  ("ragged_tails", dict(seed=31, B=2, H=2, Nq=127, Nkv=63, D=128)),
                                  ("headdim64", dict(seed=32, B=1, H=3, Nq=300, Nkv=4097, D=64))],
                         ids=["ragged_tails", "edge_127x63_d128", "edge_300x4097_d64"])
def test_race_gate_bit_identical(case):
    name, over = case
    q, k, v = make_inputs(WORKLOADS[name], **over)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    print("  race gate:", name, tuple(q.shape), tuple(k.shape), flush=True)
    ref = sage.sage_quant_prep(qd, kd, vd)
    o_ref = sage.sage_attn_fwd(ref)
    B, H, Nq, D = q.shape
    for seed in (1, 2, 3):
        got = sage.SageQuant.allocate(B, H, Nq, k.shape[2], D, dev)
        out = torch.empty_like(o_ref)
        assert _race_gate(qd, kd, vd, got, out, seed) == 0
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(ref, f).view(torch.uint8), getattr(got, f).view(torch.uint8)), (seed, f)
        assert torch.equal(o_ref.view(torch.int16), out.view(torch.int16)), seed
