"""Pins for the CPU oracle: each check ties it to something other than itself.

Kinds of pin used here: number-format definitions checked against an
independent library cast and against a table from the OCP FP8 specification;
exact rational arithmetic (fractions) for the K mean and for fma; brute-force
integer dot products for the scores; closed forms (two-pass softmax attention
in float64, online == two-pass when quantization is off); invariants (K
smoothing leaves softmax unchanged, scale equivariance, permutation
equivariance); special cases with known answers (one key, constant K); and
every rounding point of the readings recomputed exactly (fractions, mpmath's
2^x at 50 digits): INT8 ties, the multiply-by-rounded-reciprocal rules of the
INT8 and V codes, exp2 over a dense sweep and its hardest arguments, the
first tile's scores, running max, row sum and P8 codes, and the final
conversion.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import sage_oracle as so
from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.asarray(x, dtype=np.float32)


def bf16_exact(shape, rng, scale=1.0):
    """float32 array of values exactly representable in bfloat16."""
    t = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def textbook_scale(d):
    """The usual attention scale 1/sqrt(D), computed here, not by the oracle."""
    return 1.0 / math.sqrt(d)


def softmax_attention_f64(q, k, v, sm_scale):
    """Textbook softmax(Q K^T * scale) V in float64 (two passes, stable)."""
    s = (q.astype(np.float64) @ k.astype(np.float64).T) * float(sm_scale)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v.astype(np.float64)) / p.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------- formats ---

def test_e4m3_golden_table():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            val, code = line.split()[:2]
            rows.append((float(val), int(code, 16)))
    x = f32([r[0] for r in rows])
    got = so.e4m3_encode(x)
    assert [int(c) for c in got] == [r[1] for r in rows]
    # decoding the code gives back the rounded value
    dec = so.e4m3_decode(got)
    assert dec[0] == 0.0 and np.signbit(dec[1])


def test_e4m3_encode_matches_torch_cast_dense_sweep():
    # every 97th float32 bit pattern in [0, 463.99], both signs, plus all
    # midpoints between adjacent E4M3 values and their float32 neighbours
    hi = np.float32(463.99).view(np.uint32)
    bits = np.arange(0, int(hi), 97, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    vals = so.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))])
    x = np.concatenate([x, -x])
    ours = so.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = so.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.isnan(ours).sum() == 2


def test_e4m3_rejects_out_of_range():
    with pytest.raises(ValueError):
        so.e4m3_encode(f32([464.0]))


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 30, 200000))).astype(np.float32)
    # exact ties: low 16 bits == 0x8000, both parities of the kept part
    ties = (rng.integers(0x00800000, 0x7F000000, 20000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32)])
    ours = so.bf16_bits_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _round_fraction_to_f32(fr: Fraction) -> np.float32:
    cand = np.float32(float(fr))
    best = None
    for c in (np.nextafter(cand, np.float32(-np.inf)), cand, np.nextafter(cand, np.float32(np.inf))):
        dist = abs(Fraction(float(c)) - fr)
        key = (dist, int(np.float32(c).view(np.uint32)) & 1)   # ties: even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def test_fma_f32_exact_rational():
    rng = np.random.default_rng(2)
    a = f32(rng.standard_normal(3000))
    b = f32(rng.standard_normal(3000))
    c = f32(rng.standard_normal(3000) * np.exp2(rng.integers(-40, 5, 3000)))
    # constructed halfway cases: (1+2^-12)^2 = 1 + 2^-11 + 2^-24 is a float32 tie
    a = np.concatenate([a, f32([1 + 2**-12] * 3)])
    b = np.concatenate([b, f32([1 + 2**-12] * 3)])
    c = np.concatenate([c, f32([0.0, 2.0**-60, -(2.0**-60)])])
    got = so.fma_f32(a, b, c)
    for ai, bi, ci, gi in zip(a, b, c, got):
        exact = Fraction(float(ai)) * Fraction(float(bi)) + Fraction(float(ci))
        assert gi == _round_fraction_to_f32(exact), (ai, bi, ci)
    assert got[-3] == np.float32(1 + 2**-11)            # tie to even
    assert got[-2] == np.float32(1 + 2**-11 + 2**-23)   # just above the tie
    assert got[-1] == np.float32(1 + 2**-11)            # just below the tie


# ------------------------------------------------------------ quant stages --

def test_k_mean_exact_rational():
    rng = np.random.default_rng(3)
    k = bf16_exact((37, 8), rng, 3.0) + bf16_exact((1, 8), rng, 2.0)
    k = torch.from_numpy(k.astype(np.float32)).to(torch.bfloat16).float().numpy()
    ksum, mean = so.k_channel_mean(k)
    for c in range(8):
        exact = sum(Fraction(float(x)) for x in k[:, c])
        assert Fraction(float(ksum[c])) == exact
        # float64 quotient rounded to float32 equals the correctly rounded mean here
        assert mean[c] == _round_fraction_to_f32(exact / 37)


def test_k_mean_exact_rational_wide_exponents():
    """Column sums with more significant bits than float32 holds (entries from
    2^-24 to 2^4): the mean is the exact sum divided by Nkv, rounded once."""
    rng = np.random.default_rng(13)
    k = bf16_exact((53, 300), rng) * np.exp2(rng.integers(-24, 4, (53, 300))).astype(np.float32)
    ksum, mean = so.k_channel_mean(k)
    for c in range(300):
        exact = sum(Fraction(float(x)) for x in k[:, c])
        assert Fraction(float(ksum[c])) == exact
        assert mean[c] == _round_fraction_to_f32(exact / 53), c


def test_int8_block_quant_bounds_and_invariants():
    rng = np.random.default_rng(4)
    x = bf16_exact((300, 64), rng)
    x[5, 3] = 40.0  # outlier in block 0
    codes, scales = so.quantize_int8_blocks(x, 128)
    assert codes.shape == (384, 64) and scales.shape == (3,)
    assert np.all(codes[300:] == 0)
    for g in range(3):
        blk = x[g * 128:min(300, (g + 1) * 128)]
        amax = np.abs(blk).max()
        assert scales[g] == np.float32(amax) / np.float32(127)
        cb = codes[g * 128:g * 128 + blk.shape[0]].astype(np.int64)
        assert np.abs(cb).max() == 127                      # the absmax element maps to +-127
        # code is the nearest integer to x*127/A up to float32 rounding of the factor
        exact = blk.astype(np.float64) * 127.0 / float(amax)
        assert np.all(np.abs(exact - cb) <= 0.5 + 1e-5)
        assert np.all(np.sign(cb) * np.sign(blk) >= 0)
    # all-zero block: scale 0, codes 0
    z = np.zeros((64, 8), np.float32)
    c0, s0 = so.quantize_int8_blocks(z, 64)
    assert s0[0] == 0 and np.all(c0 == 0)


def test_v_fp8_channel_quant():
    rng = np.random.default_rng(5)
    v = bf16_exact((100, 16), rng)
    v[:, 7] = 0.0
    codes, vs, vamax = so.quantize_v_channels(v, 128)
    assert codes.shape == (128, 16) and np.all(codes[100:] == 0)
    assert vs[7] == 0 and np.all(codes[:, 7] == 0)
    for c in range(16):
        if c == 7:
            continue
        dec = so.e4m3_decode(codes[:100, c]) * (float(vamax[c]) / 448.0)
        # E4M3 relative spacing is 2^-3 in the normal range: error <= half a step
        rel = np.abs(dec - v[:, c]) / np.maximum(np.abs(v[:, c]), 2.0**-6 * float(vamax[c]) / 448)
        assert rel.max() <= 2.0**-4 * (1 + 1e-6)
        i = np.argmax(np.abs(v[:, c]))
        assert codes[i, c] & 0x7F == 0x7E                   # channel max maps to 448


# ----------------------------------------------------- attention pipeline --

def _tiny(nq, nkv, d, seed, bias=True, outlier=0.0):
    rng = np.random.default_rng(seed)
    q = bf16_exact((nq, d), rng)
    k = bf16_exact((nkv, d), rng) + (bf16_exact((1, d), rng, 2.0) if bias else 0)
    v = bf16_exact((nkv, d), rng)
    if outlier:
        q[rng.random((nq, d)) < outlier] *= 20
        k[rng.random((nkv, d)) < outlier] *= 20
    to = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    return to(q), to(k), to(v)


@pytest.mark.parametrize("nq,nkv,d", [(5, 7, 64), (130, 65, 64), (129, 200, 128)])
def test_scores_brute_force_int(nq, nkv, d):
    q, k, v = _tiny(nq, nkv, d, 10 + nq)
    p = so.prep_bh(q, k, v)
    rows = np.array([0, nq // 2, nq - 1])
    _, ck = so.attention_rows(p, rows, want_checkpoints=True)
    for ri, i in enumerate(rows):
        for t in range(0, nkv, 3):
            ref = sum(int(p.q_codes[i, c]) * int(p.k_codes[t, c]) for c in range(d))
            assert ck.S[ri, t] == ref
    # pad keys: zero codes give zero scores, masked to P8 = 0
    T = -(-nkv // 64)
    assert np.all(ck.P8[:, nkv:T * 64] == 0)


@pytest.mark.parametrize("nq,nkv,d", [(7, 1, 64), (64, 64, 64), (130, 200, 128), (33, 333, 64)])
def test_online_equals_two_pass_without_quantization(nq, nkv, d):
    q, k, v = _tiny(nq, nkv, d, 20 + nkv)
    p = so.prep_bh(q, k, v)
    sm = so.default_sm_scale(d)
    ob = so.attention_rows(p, None, sm, quant_qk=False, quant_p=False, quant_v=False, q_f32=q)
    got = so.bf16_bits_to_f32(ob).astype(np.float64)
    ref = softmax_attention_f64(q, k, v, float(sm))
    # float32 rounding of scores/p/RO plus one bf16 rounding of the output
    assert np.allclose(got, ref, rtol=2**-8, atol=1e-5)


def test_default_softmax_scale_literal():
    """Reading of the silent scale: 1/sqrt(D), rounded once to float32."""
    assert so.default_sm_scale(64) == np.float32(0.125)
    assert so.default_sm_scale(128) == np.float32(0.08838834764831845)
    assert so.default_sm_scale(128).dtype == np.float32


def test_k_smoothing_invariance_f64():
    q, k, v = _tiny(40, 150, 64, 31)
    sm = textbook_scale(64)
    mean = k.astype(np.float64).mean(axis=0)
    a = softmax_attention_f64(q, k, v, sm)
    b = softmax_attention_f64(q, k - mean, v, sm)
    assert np.abs(a - b).max() < 1e-12
    # and the oracle's unquantized path, which scores against smoothed K, agrees
    p = so.prep_bh(q, k, v)
    o = so.bf16_bits_to_f32(so.attention_rows(p, None, quant_qk=False, quant_p=False,
                                              quant_v=False, q_f32=q))
    assert np.allclose(o, a, rtol=2**-8, atol=1e-5)


@pytest.mark.parametrize("nq,nkv,d,outlier,bound", [
    (128, 192, 128, 0.0, 0.999), (100, 300, 64, 0.0, 0.999), (300, 1000, 128, 0.0, 0.999),
    # x20 outliers set the per-block INT8 scale, so ordinary entries keep only a
    # few bits: the method itself loses accuracy there (bound is not a pin)
    (64, 128, 128, 0.03, 0.95)])
def test_quantized_pipeline_cosine_vs_f64(nq, nkv, d, outlier, bound):
    q, k, v = _tiny(nq, nkv, d, 40 + nkv, outlier=outlier)
    p = so.prep_bh(q, k, v)
    o = so.bf16_bits_to_f32(so.attention_rows(p)).astype(np.float64).ravel()
    ref = softmax_attention_f64(q, k, v, textbook_scale(d)).ravel()
    cos = o @ ref / np.linalg.norm(o) / np.linalg.norm(ref)
    assert cos >= bound, cos


def test_quantized_pipeline_per_q_block_scales():
    """Three Q blocks (the last ragged) scaled by 1, 1/8 and 4 (exact in bf16),
    so their INT8 scales differ by those factors: each block's rows, checked on
    their own against FP64 softmax attention, stay at the method's accuracy only
    if every row is scored with its own block's scale."""
    q, k, v = _tiny(300, 200, 64, 77)
    for g, f in enumerate((1.0, 0.125, 4.0)):
        q[g * 128:(g + 1) * 128] *= f
    p = so.prep_bh(q, k, v)
    assert p.q_scale[1] * 8 < p.q_scale[0] < p.q_scale[2] / 2
    o = so.bf16_bits_to_f32(so.attention_rows(p)).astype(np.float64)
    ref = softmax_attention_f64(q, k, v, textbook_scale(64))
    for lo, hi in ((0, 64), (64, 128), (128, 192), (192, 256), (256, 300)):
        a, b = o[lo:hi].ravel(), ref[lo:hi].ravel()
        assert a @ b / np.linalg.norm(a) / np.linalg.norm(b) >= 0.995, (lo, hi)


def test_online_softmax_invariants():
    q, k, v = _tiny(50, 400, 64, 51)
    p = so.prep_bh(q, k, v)
    _, ck = so.attention_rows(p, want_checkpoints=True)
    T = ck.m.shape[1]
    assert np.all(np.diff(ck.m, axis=1) >= 0)                 # running max never decreases
    assert np.all(ck.alpha[:, 0] == 0)                         # first tile: nothing to rescale
    assert np.all((ck.alpha >= 0) & (ck.alpha <= 1))
    same = ck.m[:, 1:] == ck.m[:, :-1]
    assert np.all(ck.alpha[:, 1:][same] == 1)
    # after the tile holding the row maximum, d >= 1 (that key contributes p = 1)
    jmax = np.argmax(ck.m == ck.m[:, -1:], axis=1)
    for i in range(50):
        assert np.all(ck.d[i, jmax[i]:] >= 1)
    # the key attaining the running max of its tile gets P8 = 448 where m rose
    for i in range(50):
        for j in range(T):
            if j == 0 or ck.m[i, j] > ck.m[i, j - 1]:
                assert (ck.P8[i, j * 64:(j + 1) * 64] == 0x7E).any()


def test_single_key_special_case():
    q, k, v = _tiny(9, 1, 64, 61)
    p = so.prep_bh(q, k, v)
    o = so.bf16_bits_to_f32(so.attention_rows(p))
    # one key: p = 1, P8 = 448, d = 1, O = bf16(dec(v8) * v_scale) for every row
    deq = (so.e4m3_decode(p.v_codes[0]) * p.v_scale.astype(np.float64)).astype(np.float32)
    for i in range(9):
        assert np.allclose(o[i], deq, rtol=2**-7, atol=0)


def test_constant_k_special_case():
    rng = np.random.default_rng(71)
    q = bf16_exact((20, 64), rng)
    krow = bf16_exact((1, 64), rng)
    k = np.repeat(krow, 90, axis=0)
    v = bf16_exact((90, 64), rng)
    p = so.prep_bh(q, k, v)
    assert np.all(p.k_codes == 0) and np.all(p.k_scale == 0)
    O, ck = so.attention_rows(p, want_checkpoints=True)
    assert np.all(ck.S == 0)
    assert np.all(ck.P8[:, :90] == 0x7E) and np.all(ck.P8[:, 90:] == 0)
    mean_deq = (so.e4m3_decode(p.v_codes[:90]) * p.v_scale.astype(np.float64)).mean(axis=0)
    assert np.allclose(so.bf16_bits_to_f32(O)[0], mean_deq, rtol=2**-7, atol=1e-6)


def test_scale_and_permutation_equivariance():
    q, k, v = _tiny(128, 130, 64, 81)
    base = so.bf16_bits_to_f32(so.attention_rows(so.prep_bh(q, k, v)))
    # V * 2 -> O * 2 exactly (the per-channel scale absorbs the factor)
    o2 = so.bf16_bits_to_f32(so.attention_rows(so.prep_bh(q, k, v * 2)))
    assert np.array_equal(o2, base * 2)
    # joint permutation of channels of Q, K, V permutes O's channels
    perm = np.random.default_rng(1).permutation(64)
    op = so.bf16_bits_to_f32(so.attention_rows(so.prep_bh(q[:, perm], k[:, perm], v[:, perm])))
    assert np.array_equal(op, base[:, perm])
    # permuting query rows inside one 128-row block permutes O's rows
    rp = np.random.default_rng(2).permutation(128)
    orow = so.bf16_bits_to_f32(so.attention_rows(so.prep_bh(q[rp], k, v)))
    assert np.array_equal(orow, base[rp])


def test_kv_tile_order_matters_for_p8():
    """Strict tile order is observable: reversing K/V rows changes P8 codes."""
    q, k, v = _tiny(16, 256, 64, 91)
    _, a = so.attention_rows(so.prep_bh(q, k, v), want_checkpoints=True)
    _, b = so.attention_rows(so.prep_bh(q, k[::-1].copy(), v[::-1].copy()), want_checkpoints=True)
    assert not np.array_equal(a.P8[:, :256], b.P8[:, ::-1][:, :256])


def test_workload_inputs_reproducible_and_shaped():
    w = WORKLOADS["ragged_tails"]
    q1, k1, v1 = make_inputs(w, B=1, H=2, Nq=50, Nkv=60)
    q2, k2, v2 = make_inputs(w, B=1, H=2, Nq=50, Nkv=60)
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    assert q1.dtype == torch.bfloat16 and q1.shape == (1, 2, 50, 128)
    # K carries a per-channel bias of standard deviation about 2
    assert float(k1.float().mean(dim=2).std()) > 1.0


def test_single_tile_workload_end_to_end():
    w = WORKLOADS["single_tile"]
    q, k, v = (t[0, 0].float().numpy() for t in make_inputs(w))
    p = so.prep_bh(q, k, v)
    O, ck = so.attention_rows(p, want_checkpoints=True)
    assert O.shape == (128, 128) and ck.S.shape == (128, 192) and ck.m.shape == (128, 3)
    ref = softmax_attention_f64(q, k, v, textbook_scale(128))
    o = so.bf16_bits_to_f32(O).astype(np.float64)
    cos = (o.ravel() @ ref.ravel()) / np.linalg.norm(o) / np.linalg.norm(ref)
    assert cos >= 0.999


# ------------------------------------------- rounding points, pinned exactly --
# The readings fix the rounding of every step; the pins below compute each
# expected value with exact rational arithmetic (fractions) or 50-digit
# arithmetic (mpmath) and round it once by hand, independently of numpy's
# float32 arithmetic and of the oracle's own helpers.

def _rne_int(fr: Fraction) -> int:
    """Nearest integer to a rational, ties to even."""
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def test_int8_ties_round_half_to_even():
    """Block absmax 127, so fp32(127/A) = 1 exactly and every code is x itself
    rounded: halves go to the even neighbour (0.5 -> 0, 1.5 -> 2, 2.5 -> 2,
    126.5 -> 126)."""
    vals = [127.0, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5, 3.5, -3.5, 0.0]
    x = np.zeros((64, 16), np.float32)
    x[:len(vals), 0] = vals
    assert np.array_equal(f32(vals), torch.tensor(vals).to(torch.bfloat16).float().numpy())
    codes, scales = so.quantize_int8_blocks(x, 64)
    assert scales[0] == np.float32(1.0)
    want = [127, 0, 0, 2, -2, 2, -2, 126, -126, 4, -4, 0]
    assert [int(c) for c in codes[:len(vals), 0]] == want


def _bf16_grid(lo, hi):
    """Every positive bfloat16 value in [lo, hi), as float32."""
    a = int(np.float32(lo).view(np.uint32)) >> 16
    b = int(np.float32(hi).view(np.uint32)) >> 16
    return (np.arange(a, b, dtype=np.uint32) << 16).view(np.float32)


def _int8_cases():
    """(A, x) pairs of bf16 values where the literal rule RNE(fp32(x * fp32(127/A)))
    and the per-element division RNE(fp32(x / fp32(A/127))) give different codes
    (found with numpy float32 arithmetic; the expected codes are recomputed
    exactly below)."""
    out = []
    for A in _bf16_grid(1.0, 8.0)[::7]:
        inv = np.float32(127) / A
        sc = A / np.float32(127)
        xs = _bf16_grid(0.01, float(A))
        lit = np.rint((xs * inv).astype(np.float32))
        div = np.rint((xs / sc).astype(np.float32))
        for xv in xs[lit != div][:2]:
            out.append((float(A), float(xv)))
        if len(out) >= 12:
            break
    return out


def test_int8_code_multiplies_by_rounded_reciprocal():
    """Reading of the INT8 rule: code = RNE(fp32(x * fp32(127/A))), one
    correctly rounded reciprocal per block, not a division per element."""
    cases = _int8_cases()
    assert len(cases) >= 4
    n_div_differs = 0
    for A, xv in cases:
        blk = np.zeros((64, 4), np.float32)
        blk[0, 0], blk[1, 1], blk[2, 2] = A, xv, -xv
        codes, scales = so.quantize_int8_blocks(blk, 64)
        inv = _round_fraction_to_f32(Fraction(127) / Fraction(A))
        prod = _round_fraction_to_f32(Fraction(xv) * Fraction(float(inv)))
        want = _rne_int(Fraction(float(prod)))
        assert int(codes[1, 1]) == want and int(codes[2, 2]) == -want, (A, xv)
        assert scales[0] == _round_fraction_to_f32(Fraction(A) / 127)
        sc = _round_fraction_to_f32(Fraction(A) / 127)
        alt = _rne_int(Fraction(float(_round_fraction_to_f32(Fraction(xv) / Fraction(float(sc))))))
        n_div_differs += alt != want
    assert n_div_differs == len(cases)


def _v_cases():
    """(vamax, v) bf16 pairs where E4M3(fp32(v * fp32(448/vamax))) and
    E4M3(fp32(v / fp32(vamax/448))) differ (found with numpy float32 and torch's
    E4M3 cast)."""
    out = []
    for amax in _bf16_grid(0.5, 16.0)[::5]:
        inv = np.float32(448) / amax
        sc = amax / np.float32(448)
        vs = _bf16_grid(0.001, float(amax))
        a = torch.from_numpy((vs * inv).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        b = torch.from_numpy((vs / sc).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        for v in vs[a != b][:2]:
            out.append((float(amax), float(v)))
        if len(out) >= 12:
            break
    return out


def test_v_code_multiplies_by_rounded_reciprocal():
    """Reading of the V rule: code = E4M3_RNE(fp32(v * fp32(448/vamax))); the
    E4M3 rounding of the exactly rounded product is torch's cast."""
    cases = _v_cases()
    assert len(cases) >= 4
    for amax, v in cases:
        col = np.zeros((3, 1), np.float32)
        col[0, 0], col[1, 0], col[2, 0] = amax, v, -v
        codes, vs, _ = so.quantize_v_channels(col, 64)
        inv = _round_fraction_to_f32(Fraction(448) / Fraction(amax))
        prod = _round_fraction_to_f32(Fraction(v) * Fraction(float(inv)))
        want = torch.tensor([float(prod), -float(prod)], dtype=torch.float32).to(torch.float8_e4m3fn)
        assert [int(c) for c in codes[1:3, 0]] == want.view(torch.uint8).tolist(), (amax, v)
        assert vs[0] == _round_fraction_to_f32(Fraction(amax) / 448)
        sc = _round_fraction_to_f32(Fraction(amax) / 448)
        alt = _round_fraction_to_f32(Fraction(v) / Fraction(float(sc)))
        assert torch.tensor([float(alt)]).to(torch.float8_e4m3fn).view(torch.uint8).item() != int(codes[1, 0])


def _exp2_correct_f32(x) -> np.float32:
    """2^x at 50 digits, rounded to the nearer float32 neighbour."""
    import mpmath
    with mpmath.workdps(50):
        e = mpmath.power(2, mpmath.mpf(float(x)))
        c = np.float32(float(e))
        best = None
        for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
            key = (abs(mpmath.mpf(float(cand)) - e), int(np.float32(cand).view(np.uint32)) & 1)  # ties: even
            if best is None or key < best[0]:
                best = (key, cand)
    return np.float32(best[1])


def _exp2_hard_arguments():
    """float32 arguments whose 2^x lies closest to a float32 rounding midpoint
    (tests/golden/exp2_near_midpoint_args.txt, bit patterns; from an exhaustive
    scan of [-150, 0])."""
    with open(os.path.join(GOLDEN, "exp2_near_midpoint_args.txt")) as fh:
        bits = [int(l.split()[0], 16) for l in fh if l.strip() and not l.startswith("#")]
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_exp2_f32_correctly_rounded_against_mpmath():
    """p = fp32(2^x) correctly rounded (reading of the softmax step): a dense
    sweep of [-150, 0], random arguments and the hardest cases near midpoints."""
    rng = np.random.default_rng(9)
    x = np.concatenate([np.linspace(-150, 0, 6001, dtype=np.float32),
                        rng.uniform(-40, 0, 3000).astype(np.float32),
                        -np.exp2(rng.uniform(-30, 2, 1000)).astype(np.float32),
                        _exp2_hard_arguments()])
    got = so.exp2_f32(x)
    want = np.array([_exp2_correct_f32(v) for v in x], dtype=np.float32)
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, [(float(x[i]), float(got[i]), float(want[i])) for i in bad[:5]]
    assert so.exp2_f32(np.float32(-np.inf)) == 0 and so.exp2_f32(np.float32(0)) == 1


def _tile0_exact(p, rows, sm):
    """Tile 0 of the traversal recomputed with exact arithmetic: s, m, p, l and
    P8 for the given rows (a single-tile head, so d after tile 0 is l)."""
    import mpmath
    with mpmath.workdps(50):
        log2e = _round_fraction_to_f32(Fraction(mpmath.nstr(1 / mpmath.log(2), 45)))
    sl2 = _round_fraction_to_f32(Fraction(float(sm)) * Fraction(float(log2e)))
    nreal = min(64, p.nkv)
    out = []
    for i in rows:
        sq = p.q_scale[i // 128]
        c = _round_fraction_to_f32(Fraction(float(_round_fraction_to_f32(Fraction(float(sq)) * Fraction(float(p.k_scale[0]))))) * Fraction(float(sl2)))
        S = [sum(int(p.q_codes[i, ch]) * int(p.k_codes[t, ch]) for ch in range(p.d)) for t in range(nreal)]
        s = [_round_fraction_to_f32(Fraction(St) * Fraction(float(c))) for St in S]
        m = max(s)
        x = [_round_fraction_to_f32(Fraction(float(si)) - Fraction(float(m))) for si in s]
        pr = [_exp2_correct_f32(xi) for xi in x]
        ell = _round_fraction_to_f32(sum(Fraction(float(v)) for v in pr))
        p448 = [_round_fraction_to_f32(Fraction(float(v)) * 448) for v in pr]
        p8 = torch.tensor([float(v) for v in p448], dtype=torch.float32).to(torch.float8_e4m3fn)
        out.append((m, ell, p8.view(torch.uint8).numpy()))
    return out


@pytest.mark.parametrize("nkv", [64, 41])
def test_tile0_softmax_exact_rounding_points(nkv):
    """One 64-key tile (full, or ragged with masked keys): m, d = l (the row sum
    of the unquantized p, correctly rounded once) and the P8 codes against exact
    rational arithmetic and mpmath's 2^x, on 128 rows."""
    q, k, v = _tiny(128, nkv, 64, 300 + nkv, outlier=0.02)
    p = so.prep_bh(q, k, v)
    rows = np.arange(128)
    _, ck = so.attention_rows(p, rows, want_checkpoints=True)
    exact = _tile0_exact(p, rows, np.float32(0.125))          # 1/sqrt(64)
    for i, (m, ell, p8) in enumerate(exact):
        assert ck.m[i, 0] == m, i
        assert ck.alpha[i, 0] == 0
        assert ck.d[i, 0] == ell, (i, float(ck.d[i, 0]), float(ell))
        assert np.array_equal(ck.P8[i, :nkv], p8), i
        assert np.all(ck.P8[i, nkv:64] == 0)


def _final_order_alternatives(RO, r, vs):
    """bf16 bits of the output under the contract's rounding order and under
    three reorderings (numpy float32 arithmetic; used only to choose inputs)."""
    F32 = np.float32
    w = (vs / F32(448)).astype(F32)
    as_bf16 = lambda a: torch.from_numpy(np.asarray(a, F32)).to(torch.bfloat16).view(torch.int16).numpy()
    ref = as_bf16(((RO * r).astype(F32) * w).astype(F32))
    alts = [as_bf16((RO.astype(np.float64) * np.float64(r) * w.astype(np.float64)).astype(F32)),
            as_bf16((RO * (r * w).astype(F32)).astype(F32)),
            as_bf16(((RO * (F32(1) / (F32(1) / r * F32(448))).astype(F32)).astype(F32) * vs).astype(F32))]
    return ref, alts


def test_final_conversion_rounding_points():
    """Constant K: every real key scores 0, so p = 1, d = n, P8 = 448 and
    RO = fp32(448 * sum_t dec(V8[t, c])) (the exact tile sum rounded once).  The
    output must be bf16(fp32(fp32(RO * fp32(1/d)) * fp32(v_scale/448))), checked
    with exact rationals on a wide head whose seed is chosen (numpy search) so
    that three reorderings of the final scaling change some bf16 outputs."""
    n, D = 3, 4096
    for seed in range(200):
        rng = np.random.default_rng(1000 + seed)
        v = bf16_exact((n, D), rng)
        codes, vs, _ = so.quantize_v_channels(v, 64)   # choosing the inputs only
        RO = (448.0 * so.e4m3_decode(codes[:n]).sum(axis=0)).astype(np.float32)
        ref, alts = _final_order_alternatives(RO, np.float32(1) / np.float32(n), vs)
        if all((a != ref).any() for a in alts):
            break
    else:
        pytest.fail("no discriminating input found")
    k = np.repeat(bf16_exact((1, D), rng), n, axis=0)
    q = bf16_exact((2, D), rng)
    p = so.prep_bh(q, k, v)
    assert np.all(p.k_codes == 0)
    O, ck = so.attention_rows(p, want_checkpoints=True)
    r = _round_fraction_to_f32(Fraction(1, n))
    want = np.zeros(D, np.float32)
    for c in range(D):
        ro = _round_fraction_to_f32(sum(Fraction(448) * Fraction(float(x)) for x in so.e4m3_decode(p.v_codes[:n, c])))
        assert ck.RO[0, c] == ro
        w = _round_fraction_to_f32(Fraction(float(p.v_scale[c])) / 448)
        want[c] = _round_fraction_to_f32(Fraction(float(_round_fraction_to_f32(Fraction(float(ro)) * Fraction(float(r))))) * Fraction(float(w)))
    assert ck.r[0] == r
    want_bits = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O[0], want_bits) and np.array_equal(O[1], want_bits)
