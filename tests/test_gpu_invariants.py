"""GPU-path invariants that hold exactly, plus graph capture and repetition.

Exact by construction of the method (and so bit-exact on the GPU too):
  * V * 2 -> O * 2 (the per-channel V scale absorbs the factor exactly);
  * a joint permutation of the channels of Q, K, V permutes O's channels
    (integer scores are exact; each output channel sees the same products);
  * a permutation of query rows inside one 128-row block permutes O's rows.
Determinism: repeated launches give identical bytes (the pages' prototype was
checked over 1,000 launches, "Experiment Log", Phase 2B).
Graph capture: prep + forward captured once and replayed gives the eager
result every time (the library allocates nothing and never synchronizes).
"""

import numpy as np
import pytest
import torch

from quantized_exact_attention_amd import sage
from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(q, k, v, sm_scale=None):
    return sage.sage_attention(q.to(DEV), k.to(DEV), v.to(DEV), sm_scale).cpu()


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("D", [64, 128])
def test_v_times_two_doubles_output_exactly(D):
    q, k, v = make_inputs(WORKLOADS["ragged_tails"], seed=11, B=1, H=2, Nq=300, Nkv=500, D=D)
    a = _run(q, k, v)
    b = _run(q, k, v * 2)
    assert torch.equal(_bits(b), _bits(a * 2))


@pytest.mark.parametrize("D", [64, 128])
def test_channel_permutation_equivariance(D):
    q, k, v = make_inputs(WORKLOADS["ragged_tails"], seed=12, B=1, H=2, Nq=260, Nkv=333, D=D)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(D))
    a = _run(q, k, v)
    b = _run(q[..., perm].contiguous(), k[..., perm].contiguous(), v[..., perm].contiguous())
    assert torch.equal(_bits(b), _bits(a[..., perm].contiguous()))


def test_row_permutation_inside_a_block():
    q, k, v = make_inputs(WORKLOADS["dit_block"], seed=13, B=1, H=1, Nq=256, Nkv=700, D=128)
    rp = torch.cat([torch.from_numpy(np.random.default_rng(4).permutation(128)),
                    128 + torch.from_numpy(np.random.default_rng(5).permutation(128))])
    a = _run(q, k, v)
    b = _run(q[:, :, rp].contiguous(), k, v)
    assert torch.equal(_bits(b), _bits(a[:, :, rp].contiguous()))


def test_strided_output_view():
    q, k, v = make_inputs(WORKLOADS["ragged_tails"], seed=14, B=2, H=3, Nq=150, Nkv=90, D=128)
    quant = sage.sage_quant_prep(q.to(DEV), k.to(DEV), v.to(DEV))
    dense = sage.sage_attn_fwd(quant)
    store = torch.zeros(2, 150, 3, 128, dtype=torch.bfloat16, device=DEV)   # [B,N,H,D] memory
    view = store.transpose(1, 2)
    sage.sage_attn_fwd(quant, out=view)
    assert torch.equal(_bits(view.contiguous()), _bits(dense.contiguous()))


def test_thousand_launches_bit_identical():
    q, k, v = make_inputs(WORKLOADS["ragged_tails"])
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    quant = sage.sage_quant_prep(qd, kd, vd)
    first = sage.sage_attn_fwd(quant).clone()
    out = torch.empty_like(first)
    mismatches = torch.zeros((), dtype=torch.int64, device=DEV)
    for i in range(1000):
        if i % 10 == 0:
            sage.sage_quant_prep(qd, kd, vd, out=quant)
        sage.sage_attn_fwd(quant, out=out)
        mismatches += (_bits(out) != _bits(first)).sum()
    torch.cuda.synchronize()
    assert int(mismatches) == 0


@pytest.mark.parametrize("mode", ["three_launches", "single_pass", "q_quantizing_pair"])
def test_graph_capture_replay_matches_eager(mode):
    w = WORKLOADS["ragged_tails"]
    q, k, v = make_inputs(w, seed=21, B=1, H=4, Nq=500, Nkv=700, D=128)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    single_pass = mode == "single_pass"
    if mode == "q_quantizing_pair":
        quant = sage.sage_quant_prep_kv(kd, vd)
        out = sage.sage_attn_fwd_q(qd, quant)
    else:
        quant = sage.sage_quant_prep(qd, kd, vd, single_pass=single_pass)
        out = sage.sage_attn_fwd(quant)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            if mode == "q_quantizing_pair":
                sage.sage_quant_prep_kv(kd, vd, out=quant)
                sage.sage_attn_fwd_q(qd, quant, out=out)
            else:
                sage.sage_quant_prep(qd, kd, vd, out=quant, single_pass=single_pass)
                sage.sage_attn_fwd(quant, out=out)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(4):
        # new inputs written in place, then replay, then compare with an eager run
        q2, k2, v2 = make_inputs(w, seed=100 + r, B=1, H=4, Nq=500, Nkv=700, D=128)
        qd.copy_(q2.to(DEV))
        kd.copy_(k2.to(DEV))
        vd.copy_(v2.to(DEV))
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        eager = sage.sage_attention(qd, kd, vd)
        torch.cuda.synchronize()
        assert torch.equal(_bits(replayed), _bits(eager)), "replay %d differs" % r


def test_binding_rejects_mismatched_buffers():
    """The binding checks, before any launch, that a reused quantized set and
    an output fit the call: same shape, same device, large enough, and an
    output whose rows do not overlap (the C ABI's SAGE_E_ALIAS)."""
    q, k, v = (t.to(DEV) for t in make_inputs(WORKLOADS["ragged_tails"], seed=5, B=1, H=2, Nq=130, Nkv=200, D=64))
    quant = sage.sage_quant_prep(q, k, v)
    with pytest.raises(ValueError, match="another shape"):
        sage.sage_quant_prep(q[:, :, :100], k, v, out=quant)
    small = sage.SageQuant.allocate(1, 2, 130, 200, 64, DEV)
    small.k_codes = small.k_codes[:-64]
    with pytest.raises(ValueError, match="smaller"):
        sage.sage_quant_prep(q, k, v, out=small)
    with pytest.raises(ValueError, match="device"):
        sage.sage_attn_fwd(quant, out=torch.empty(1, 2, 130, 64, dtype=torch.bfloat16))
    base = torch.empty(130 * 64, dtype=torch.bfloat16, device=DEV)
    aliased = base.as_strided((1, 2, 130, 64), (0, 0, 64, 1))          # both heads on one block
    with pytest.raises(sage.SageError, match="SAGE_E_ALIAS"):
        sage.sage_attn_fwd(quant, out=aliased)
    torch.cuda.synchronize()
    ref = sage.sage_attn_fwd(quant)
    assert torch.equal(sage.sage_attn_fwd(quant), ref)                  # the set is still usable


@pytest.mark.parametrize("mode", ["three_launches", "single_pass", "q_quantizing_pair"])
def test_calls_with_preallocated_buffers_allocate_nothing(mode):
    """With the quantized set and the output passed in, prep + forward make no
    device allocation (torch's allocator counts every request, cached or not):
    the path a captured graph or an allocation-free caller relies on."""
    q, k, v = (t.to(DEV) for t in make_inputs(WORKLOADS["ragged_tails"], seed=8, B=1, H=3, Nq=200, Nkv=300, D=128))
    single_pass = mode == "single_pass"
    pair = mode == "q_quantizing_pair"
    quant = sage.sage_quant_prep_kv(k, v) if pair else sage.sage_quant_prep(q, k, v, single_pass=single_pass)
    out = sage.sage_attn_fwd_q(q, quant) if pair else sage.sage_attn_fwd(quant)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats(DEV)["allocation.all.allocated"]
    for _ in range(3):
        if pair:
            sage.sage_quant_prep_kv(k, v, out=quant)
            sage.sage_attn_fwd_q(q, quant, out=out)
        else:
            sage.sage_quant_prep(q, k, v, out=quant, single_pass=single_pass)
            sage.sage_attn_fwd(quant, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats(DEV)["allocation.all.allocated"] == before
    assert torch.equal(_bits(out), _bits(sage.sage_attention(q, k, v)))


def test_two_streams_at_once_match_sequential_runs():
    """The library keeps no per-call state: prep + forward of two independent
    problems enqueued on two streams at the same time (default priority) give
    the sequential results bit for bit (the three-launch prep; the single pass
    must not share the device with other work, as its header says)."""
    w = WORKLOADS["ragged_tails"]
    a = [t.to(DEV) for t in make_inputs(w, seed=31, B=1, H=4, Nq=700, Nkv=900, D=128)]
    b = [t.to(DEV) for t in make_inputs(w, seed=32, B=2, H=2, Nq=500, Nkv=1300, D=64)]
    ref_a = sage.sage_attn_fwd(sage.sage_quant_prep(*a))
    ref_b = sage.sage_attn_fwd(sage.sage_quant_prep(*b))
    qa, qb = sage.sage_quant_prep(*a), sage.sage_quant_prep(*b)
    oa, ob = torch.empty_like(ref_a), torch.empty_like(ref_b)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(5):
        with torch.cuda.stream(sa):
            sage.sage_quant_prep(*a, out=qa)
            sage.sage_attn_fwd(qa, out=oa)
        with torch.cuda.stream(sb):
            sage.sage_quant_prep(*b, out=qb)
            sage.sage_attn_fwd(qb, out=ob)
    torch.cuda.synchronize()
    assert torch.equal(_bits(oa), _bits(ref_a)) and torch.equal(_bits(ob), _bits(ref_b))
