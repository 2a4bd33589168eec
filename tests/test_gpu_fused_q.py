"""The K/V-only prep and the Q-quantizing forward on the GPU.

sage_quant_prep_kv must write the K/V half of sage_quant_prep bit for bit, and
sage_attn_fwd_q (each workgroup quantizes its own Q block by the prep's rule)
must give the output of sage_quant_prep + sage_attn_fwd bit for bit, on ragged
and full-size shapes, both head dimensions, strided Q, and a K/V set reused for
queries of other lengths.  Rows are also held against the oracle directly.
"""

import numpy as np
import pytest
import torch

from oracle import sage_oracle as so
from quantized_exact_attention_amd import sage
from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs
from tests import test_gpu_parity as tp

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sage.lib()


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def _kv_equal(a, b):
    for name in ("k_mean", "k_codes", "k_scale", "v_codes", "v_scale"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), name


CASES = [
    # (B, H, Nq, Nkv, D, seed)
    (1, 3, 1, 1, 128, 1), (1, 2, 129, 65, 64, 2), (2, 2, 300, 777, 128, 3), (1, 4, 1000, 1000, 64, 4),
    (1, 1, 5, 4097, 128, 5), (2, 3, 255, 130, 128, 6),
]


@pytest.mark.parametrize("B,H,Nq,Nkv,D,seed", CASES)
def test_kv_prep_and_q_quantizing_forward_match_the_two_calls(B, H, Nq, Nkv, D, seed):
    q, k, v = make_inputs(WORKLOADS["ragged_tails"], seed=seed, B=B, H=H, Nq=Nq, Nkv=Nkv, D=D)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    print("  fused-Q case B=%d H=%d Nq=%d Nkv=%d D=%d" % (B, H, Nq, Nkv, D), flush=True)
    full = sage.sage_quant_prep(qd, kd, vd)
    ref = sage.sage_attn_fwd(full)
    kv = sage.sage_quant_prep_kv(kd, vd)
    assert kv.kv_only
    out = sage.sage_attn_fwd_q(qd, kv)
    out_full_set = sage.sage_attn_fwd_q(qd, full)          # a complete set serves too
    torch.cuda.synchronize()
    _kv_equal(kv, full)
    assert np.array_equal(_bits(out), _bits(ref))
    assert np.array_equal(_bits(out_full_set), _bits(ref))
    with pytest.raises(ValueError):
        sage.sage_attn_fwd(kv)                              # the two-call forward needs the Q codes


def test_strided_q_custom_scale_and_preallocated_output():
    q, k, v = make_inputs(WORKLOADS["ragged_tails"], seed=7, B=2, H=3, Nq=400, Nkv=300, D=128)
    # [B,N,H,D] storage viewed as [B,H,N,D]
    qd = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    kd, vd = k.to(DEV), v.to(DEV)
    ref = sage.sage_attn_fwd(sage.sage_quant_prep(qd, kd, vd), 0.05)
    kv = sage.sage_quant_prep_kv(kd, vd)
    out = torch.empty(2, 400, 3, 128, dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    got = sage.sage_attn_fwd_q(qd, kv, 0.05, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert np.array_equal(_bits(got.contiguous()), _bits(ref))


def test_one_kv_set_serves_queries_of_other_lengths():
    """K/V prepared once; queries of 300 and 1000 rows against it each give the
    two-call result for their own (q, k, v)."""
    w = WORKLOADS["ragged_tails"]
    _, k, v = make_inputs(w, seed=8, B=1, H=4, Nq=8, Nkv=900, D=64)
    kd, vd = k.to(DEV), v.to(DEV)
    kv = sage.sage_quant_prep_kv(kd, vd)
    for nq, seed in ((300, 9), (1000, 10), (1, 11)):
        q, _, _ = make_inputs(w, seed=seed, B=1, H=4, Nq=nq, Nkv=900, D=64)
        qd = q.to(DEV)
        got = sage.sage_attn_fwd_q(qd, kv)
        ref = sage.sage_attn_fwd(sage.sage_quant_prep(qd, kd, vd))
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(ref)), nq


def test_q_quantizing_forward_against_the_oracle():
    """Every row of one ragged head against the oracle (same bar as the parity tests)."""
    q, k, v = make_inputs(WORKLOADS["ragged_tails"], seed=12, B=1, H=2, Nq=333, Nkv=500, D=128)
    got = sage.sage_attn_fwd_q(q.to(DEV), sage.sage_quant_prep_kv(k.to(DEV), v.to(DEV)))
    O = got.view(torch.int16).cpu().numpy().view(np.uint16)
    stats = tp.OStats()
    for h in range(2):
        p = so.prep_bh(q[0, h].float().numpy(), k[0, h].float().numpy(), v[0, h].float().numpy())
        O_ref = so.attention_rows(p, np.arange(333))
        stats.add_o(O[0, h], O_ref)
    stats.check()


@pytest.mark.parametrize("name", ["dit_block", "long_video", "headdim64"])
def test_full_size_bit_identical(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    del q, k, v
    print("  fused-Q full size %s" % name, flush=True)
    ref = sage.sage_attn_fwd(sage.sage_quant_prep(qd, kd, vd))
    kv = sage.sage_quant_prep_kv(kd, vd)
    got = sage.sage_attn_fwd_q(qd, kv)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    del ref, got, kv
    torch.cuda.empty_cache()


def _sweep_cases(n=40):
    rng = np.random.default_rng(77)
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
        Nq, Nkv = int(rng.integers(1, 1500)), int(rng.integers(1, 1500))
        dist = str(rng.choice(["dit_block", "ragged_tails", "headdim64"]))   # no / 3% / 1% outliers
        sm = None if rng.random() < 0.7 else float(rng.uniform(0.02, 0.3))
        strided = bool(rng.random() < 0.3)
        cases.append((i, dist, B, H, Nq, Nkv, D, sm, strided))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "s%d_%s_%dx%dx%dx%dx%d" % (c[0], c[1], *c[2:7]))
def test_random_shapes_bit_identical_to_the_two_calls(case):
    i, dist, B, H, Nq, Nkv, D, sm, strided = case
    q, k, v = make_inputs(WORKLOADS[dist], seed=500 + i, B=B, H=H, Nq=Nq, Nkv=Nkv, D=D)
    if strided:
        qd, kd, vd = (t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v))
    else:
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref = sage.sage_attn_fwd(sage.sage_quant_prep(qd, kd, vd), sm)
    got = sage.sage_attn_fwd_q(qd, sage.sage_quant_prep_kv(kd, vd), sm)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(got), _bits(ref))
