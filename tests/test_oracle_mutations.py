"""Planted mistakes in the oracle are caught by its pins.

Each case edits one expression in the text of ``oracle/sage_oracle.py`` (a
wrong sign, a dropped term, a transposed operand, a wrong constant, index or
rounding), loads the edited text as a separate module and runs the pins of
``tests/test_oracle_pins.py`` against it, cheapest first, until one fails.  A
mutant that passes every pin would mean the pins cannot tell that mistake from
the method.  The oracle itself is never modified.
"""

import inspect
import sys
import types

import numpy as np
import pytest

import oracle.sage_oracle as real
from tests import test_oracle_pins as pins

# (name, exact text in the oracle, replacement)
MUTATIONS = [
    # number formats
    ("e4m3 rounds half away from zero", "q = np.rint(a / quantum)", "q = np.floor(a / quantum + 0.5)"),
    ("e4m3 mantissa field off by one", "code = np.where(sub, code, (re + 7) * 8 + mant)",
     "code = np.where(sub, code, (re + 8) * 8 + mant)"),
    ("e4m3 decode bias", "(1.0 + m / 8.0) * np.ldexp(1.0, e - 7)", "(1.0 + m / 8.0) * np.ldexp(1.0, e - 8)"),
    ("bf16 truncates", "r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16", "r = u >> 16"),
    ("fma rounds twice", "return np.where(midpoint, np.where(err > 0, hi, lo), r).astype(F32)",
     "return ((a * b).astype(F32) + c.astype(F32)).astype(F32)"),
    # prep
    ("K mean divided by Nkv-1", "mean = (ksum / F64(k.shape[0])).astype(F32)",
     "mean = (ksum / F64(max(1, k.shape[0] - 1))).astype(F32)"),
    ("K smoothing sign", "ks = (k - mean[None, :]).astype(F32)", "ks = (k + mean[None, :]).astype(F32)"),
    ("Q smoothed too", "qc, qs = quantize_int8_blocks(q, BQ)",
     "qc, qs = quantize_int8_blocks((q - q.mean(axis=0)[None, :]).astype(F32), BQ)"),
    ("INT8 scale divisor", "scales[g] = amax / F32(QMAX)", "scales[g] = amax / F32(128)"),
    ("INT8 rounding truncates", "q = np.rint((blk * inv).astype(F32))", "q = np.trunc((blk * inv).astype(F32))"),
    ("Q block size 64", "qc, qs = quantize_int8_blocks(q, BQ)", "qc, qs = quantize_int8_blocks(q, BK)"),
    ("V scale divisor", "vscale = np.where(vamax == 0, F32(0), safe / F32(F8MAX)).astype(F32)",
     "vscale = np.where(vamax == 0, F32(0), safe / F32(256)).astype(F32)"),
    ("V max over keys of the first tile only", "vamax = np.abs(v).max(axis=0).astype(F32)",
     "vamax = np.abs(v[:64]).max(axis=0).astype(F32)"),
    # traversal
    ("K operand not transposed", "S = qc @ p.k_codes[k0:k0 + BK].astype(F64).T",
     "S = qc @ p.k_codes[k0:k0 + BK].astype(F64)"),
    ("k scale of tile 0", "cj = F32(F32(sq * p.k_scale[j]) * sl2)", "cj = F32(F32(sq * p.k_scale[0]) * sl2)"),
    ("log2 e not folded", "sl2 = F32(sm * LOG2E_F32)", "sl2 = F32(sm)"),
    ("softmax scale 1/D", "return F32(1.0 / np.sqrt(F64(d)))", "return F32(1.0 / F64(d))"),
    ("ragged keys not masked", "s[:, nreal:] = -np.inf", "s[:, nreal:] = s[:, nreal:]"),
    ("running max not carried", "m_new = np.maximum(m, s.max(axis=1))", "m_new = s.max(axis=1)"),
    ("exp base e", "pr = exp2_f32(x)", "pr = np.exp(x.astype(F64)).astype(F32)"),
    ("d without rescale", "dsum = fma_f32(dsum, alpha, ell)", "dsum = (dsum + ell).astype(F32)"),
    ("d from the FP8 codes", "ell = pr.astype(F64).sum(axis=1).astype(F32)",
     "ell = (e4m3_decode(e4m3_encode((pr * F32(F8MAX)).astype(F32))) / F8MAX).sum(axis=1).astype(F32)"),
    ("P scale 256", "p8 = e4m3_encode((pr * F32(F8MAX)).astype(F32))", "p8 = e4m3_encode((pr * F32(256)).astype(F32))"),
    ("V operand transposed", "partial = (pd @ vd).astype(F32)", "partial = (pd @ vd.T).astype(F32)"),
    ("RO without rescale", "RO = fma_f32(RO, alpha[:, None], partial)", "RO = (RO + partial).astype(F32)"),
    ("V scale left out of the output", "w = (p.v_scale / F32(F8MAX)).astype(F32)",
     "w = np.full_like(p.v_scale, F32(1) / F32(F8MAX))"),
    ("reciprocal of the first row's d", "r = (F32(1) / dsum).astype(F32)",
     "r = np.full_like(dsum, F32(1) / dsum[0])"),
    ("V inverse inverted", "inv = np.where(vamax == 0, F32(0), F32(F8MAX) / safe).astype(F32)",
     "inv = np.where(vamax == 0, F32(0), safe / F32(F8MAX)).astype(F32)"),
    ("rescale exponent sign", "alpha = exp2_f32((m - m_new).astype(F32))", "alpha = exp2_f32((m_new - m).astype(F32))"),
    ("p against the old max", "x = (s - m_new[:, None]).astype(F32)", "x = (s - np.maximum(m, F32(-1e30))[:, None]).astype(F32)"),
    ("output divided by the reciprocal", "o32 = ((RO * r[:, None]).astype(F32) * w[None, :]).astype(F32)",
     "o32 = ((RO / r[:, None]).astype(F32) * w[None, :]).astype(F32)"),
    ("K mean taken from Q", "ksum, mean = k_channel_mean(k)", "ksum, mean = k_channel_mean(q)"),
    ("V max without abs", "vamax = np.abs(v).max(axis=0).astype(F32)", "vamax = v.max(axis=0).astype(F32)"),
    ("q scale of the wrong block", "sq = p.q_scale[rows // BQ]", "sq = p.q_scale[np.minimum(rows // BK, p.q_scale.size - 1)]"),
    ("tiles in reverse order", "for j in range(T):", "for j in reversed(range(T)):"),
    ("row sum over half the tile", "ell = pr.astype(F64).sum(axis=1).astype(F32)",
     "ell = pr[:, :32].astype(F64).sum(axis=1).astype(F32)"),
    ("e4m3 subnormal quantum", "code = np.where(sub, np.rint(r / 2.0 ** -9), code)",
     "code = np.where(sub, np.rint(r / 2.0 ** -10), code)"),
    ("INT8 absmax over the whole tensor", "amax = F32(np.abs(blk).max())", "amax = F32(np.abs(x).max())"),
    # rounding points of the readings
    ("INT8 ties away from zero", "q = np.rint((blk * inv).astype(F32))",
     "q = np.sign(blk) * np.floor(np.abs((blk * inv).astype(F32)) + F32(0.5))"),
    ("INT8 code by per-element division", "q = np.rint((blk * inv).astype(F32))",
     "q = np.rint((blk / scales[g]).astype(F32))"),
    ("V code by per-element division", "codes[:n] = e4m3_encode((v * inv[None, :]).astype(F32))",
     "codes[:n] = e4m3_encode((v / np.where(vscale == 0, F32(1), vscale)[None, :]).astype(F32))"),
    ("exp2 evaluated in float32", "y = np.exp2(xf.astype(F64))", "y = np.exp2(xf).astype(F64)"),
    ("exp2 without the near-midpoint refinement", "if np.any(near):", "if False:"),
    ("row sum in float32", "ell = pr.astype(F64).sum(axis=1).astype(F32)", "ell = pr.sum(axis=1, dtype=F32)"),
    ("score factor rounded once", "cj = F32(F32(sq * p.k_scale[j]) * sl2)",
     "cj = (sq.astype(F64) * F64(p.k_scale[j]) * F64(sl2)).astype(F32)"),
    ("exp2 argument rounded once", "x = (s - m_new[:, None]).astype(F32)",
     "x = (S.astype(F64) * cj[:, None].astype(F64) - m_new[:, None].astype(F64)).astype(F32)"),
    ("output scaled in one rounding", "o32 = ((RO * r[:, None]).astype(F32) * w[None, :]).astype(F32)",
     "o32 = (RO.astype(F64) * r[:, None].astype(F64) * w[None, :].astype(F64)).astype(F32)"),
    ("output scale folded before the reciprocal", "o32 = ((RO * r[:, None]).astype(F32) * w[None, :]).astype(F32)",
     "o32 = (RO * (r[:, None] * w[None, :]).astype(F32)).astype(F32)"),
    ("partial added before the rescale", "RO = fma_f32(RO, alpha[:, None], partial)",
     "RO = ((RO + partial) * alpha[:, None]).astype(F32)"),
    ("K mean divided in float32", "mean = (ksum / F64(k.shape[0])).astype(F32)",
     "mean = (ksum.astype(F32) / F32(k.shape[0])).astype(F32)"),
    ("1/448 folded into the reciprocal", "r = (F32(1) / dsum).astype(F32)",
     "r = (F32(1) / (dsum * F32(F8MAX))).astype(F32); w = p.v_scale"),
]

# The pins, cheapest first (parametrized pins with one or two of their cases).
PINS = [
    ("e4m3 golden table", pins.test_e4m3_golden_table),
    ("softmax scale literal", pins.test_default_softmax_scale_literal),
    ("e4m3 decode", pins.test_e4m3_decode_all_codes_matches_torch),
    ("bf16 rne", pins.test_bf16_rne_matches_torch_cast),
    ("fma exact", pins.test_fma_f32_exact_rational),
    ("k mean exact", pins.test_k_mean_exact_rational),
    ("k mean exact, wide exponents", pins.test_k_mean_exact_rational_wide_exponents),
    ("int8 invariants", pins.test_int8_block_quant_bounds_and_invariants),
    ("v fp8", pins.test_v_fp8_channel_quant),
    ("scores 5x7", lambda: pins.test_scores_brute_force_int(5, 7, 64)),
    ("scores 130x65", lambda: pins.test_scores_brute_force_int(130, 65, 64)),
    ("single key", pins.test_single_key_special_case),
    ("constant k", pins.test_constant_k_special_case),
    ("online == two-pass 64", lambda: pins.test_online_equals_two_pass_without_quantization(64, 64, 64)),
    ("online == two-pass 33x333", lambda: pins.test_online_equals_two_pass_without_quantization(33, 333, 64)),
    ("k smoothing", pins.test_k_smoothing_invariance_f64),
    ("softmax invariants", pins.test_online_softmax_invariants),
    ("equivariance", pins.test_scale_and_permutation_equivariance),
    ("cosine 128x192", lambda: pins.test_quantized_pipeline_cosine_vs_f64(128, 192, 128, 0.0, 0.999)),
    ("per-block Q scales", pins.test_quantized_pipeline_per_q_block_scales),
    ("single tile end to end", pins.test_single_tile_workload_end_to_end),
    ("e4m3 dense sweep", pins.test_e4m3_encode_matches_torch_cast_dense_sweep),
    ("int8 ties", pins.test_int8_ties_round_half_to_even),
    ("int8 reciprocal rule", pins.test_int8_code_multiplies_by_rounded_reciprocal),
    ("v reciprocal rule", pins.test_v_code_multiplies_by_rounded_reciprocal),
    ("exp2 vs mpmath", pins.test_exp2_f32_correctly_rounded_against_mpmath),
    ("tile 0 exact, full", lambda: pins.test_tile0_softmax_exact_rounding_points(64)),
    ("tile 0 exact, ragged", lambda: pins.test_tile0_softmax_exact_rounding_points(41)),
    ("final conversion exact", pins.test_final_conversion_rounding_points),
]


def _mutant(old, new):
    src = inspect.getsource(real)
    assert src.count(old) == 1, "mutation anchor must occur exactly once: %r" % old
    name = "sage_oracle_mutant"
    mod = types.ModuleType(name)
    mod.__file__ = real.__file__
    sys.modules[name] = mod                     # dataclasses look their module up
    try:
        exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    except Exception:
        sys.modules.pop(name, None)
        raise
    return mod


def test_unmutated_oracle_passes_the_pin_list():
    for _, pin in PINS[:13]:
        pin()


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, monkeypatch):
    mod = _mutant(old, new)
    monkeypatch.setattr(pins, "so", mod)
    caught = None
    with np.errstate(all="ignore"):
        for pin_name, pin in PINS:
            try:
                pin()
            except Exception:                   # an assertion, or the mutant crashing
                caught = pin_name
                break
    sys.modules.pop("sage_oracle_mutant", None)
    assert caught is not None, "no pin catches the planted mistake: %s" % name
