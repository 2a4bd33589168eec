"""The GPU parity comparison, tested on the CPU with planted mistakes.

The comparison functions of tests/test_gpu_parity.py hold the library's
buffers against the oracle.  Here a stand-in for those buffers is built from
the oracle's own results (in the library's layouts where the comparison reads
them), so the unmodified stand-in must pass every check; then one mistake at a
time is planted in the stand-in (one code, one scale, one score, one
checkpoint, one output entry) and the comparison must fail, naming the stage.
This is host fault injection done without a GPU: the repetition test of
"Experiment Log", Phase 2B, found a slot-indexing bug on the pages' machine,
and the comparison must be able to see such a mistake at every stage.
"""

import copy

import numpy as np
import pytest

from oracle import sage_oracle as so
from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs
from tests import test_gpu_parity as tp

B, H, NQ, NKV, D = 1, 2, 130, 200, 64          # two Q blocks (second ragged), four K tiles (last ragged)


class _Quant:
    def __init__(self, nqb, T):
        self.nqb, self.T = nqb, T


class OracleStandIn:
    """The attributes of tests/test_gpu_parity.Run that the comparison reads,
    filled from the oracle: prep outputs, the forward's output bits and the
    capture buffers of every unit (rows padded to 128, keys to T*64)."""

    def __init__(self):
        q, k, v = make_inputs(WORKLOADS["ragged_tails"], seed=5, B=B, H=H, Nq=NQ, Nkv=NKV, D=D)
        self.q, self.k, self.v = q, k, v
        self.B, self.H, self.Nq, self.Nkv, self.D = B, H, NQ, NKV, D
        self.sm_scale = None
        nqb, T = -(-NQ // 128), -(-NKV // 64)
        self.quant = _Quant(nqb, T)
        self.units = list(range(B * H * nqb))
        BH = B * H
        self.preps = [so.prep_bh(q[b, h].float().numpy(), k[b, h].float().numpy(), v[b, h].float().numpy())
                      for b in range(B) for h in range(H)]
        self.k_mean = np.stack([p.k_mean for p in self.preps])
        self.q_scale = np.stack([p.q_scale for p in self.preps])
        self.k_scale = np.stack([p.k_scale for p in self.preps])
        self.v_scale = np.stack([p.v_scale for p in self.preps])
        self._codes = [(p.q_codes.copy(), p.k_codes.copy(), p.v_codes.copy()) for p in self.preps]
        n = len(self.units)
        self.O = np.zeros((B, H, NQ, D), np.uint16)
        self.S = np.zeros((n, 128, T * 64), np.int32)
        self.P8 = np.zeros((n, 128, T * 64), np.uint8)
        self.MD = np.zeros((n, 128, T, 3), np.float32)
        self.PART = np.zeros((n, 128, T, D), np.float32)
        self.RO = np.zeros((n, 128, T, D), np.float32)
        self.R = np.zeros((n, 128), np.float32)
        for ci, u in enumerate(self.units):
            bh, qb = divmod(u, nqb)
            b, h = divmod(bh, H)
            rows = np.arange(qb * 128, min(NQ, (qb + 1) * 128))
            nr = rows.size
            O_ref, ck = so.attention_rows(self.preps[bh], rows, None, want_checkpoints=True)
            self.O[b, h, rows] = O_ref
            self.S[ci, :nr] = ck.S
            self.P8[ci, :nr] = ck.P8
            self.MD[ci, :nr, :, 0] = ck.m
            self.MD[ci, :nr, :, 1] = (ck.d.astype(np.float64) * 448.0).astype(np.float32)
            self.MD[ci, :nr, :, 2] = ck.alpha
            self.PART[ci, :nr] = ck.partial
            self.RO[ci, :nr] = ck.RO_tiles
            self.R[ci, :nr] = (ck.r.astype(np.float64) / 448.0).astype(np.float32)
        self.Oc = self.O.copy()

    def codes(self, bh):
        return self._codes[bh]

    def oracle_prep(self, bh):
        return self.preps[bh]


@pytest.fixture(scope="module")
def clean():
    return OracleStandIn()


def _check_all(run):
    for bh in range(run.B * run.H):
        tp.check_prep_bh(run, bh, run.preps[bh])
    stats = tp.OStats()
    tp.check_units(run, stats, {bh: run.preps[bh] for bh in range(run.B * run.H)})
    stats.check(tp.O_OVER_FRAC_GAUSSIAN)


def test_comparison_accepts_the_oracle_itself(clean):
    _check_all(clean)


def _plant(clean, what):
    run = copy.deepcopy(clean)
    bh = 1
    if what == "k_mean":
        run.k_mean[bh, 3] = np.nextafter(run.k_mean[bh, 3], np.float32(np.inf))
    elif what == "q_scale":
        run.q_scale[bh, 1] *= np.float32(2)
    elif what == "k_scale":
        run.k_scale[bh, 3] = np.nextafter(run.k_scale[bh, 3], np.float32(0))
    elif what == "v_scale":
        run.v_scale[bh, 10] = np.nextafter(run.v_scale[bh, 10], np.float32(np.inf))
    elif what in ("q codes", "k codes", "v codes"):
        qc, kc, vc = run._codes[bh]
        arr = {"q codes": qc, "k codes": kc, "v codes": vc}[what]
        arr[129, 7] = arr[129, 7] ^ 1          # one bit of one code, in the ragged last block
    elif what == "S mismatch":
        run.S[2, 50, 130] += 1
    elif what == "m mismatch":
        run.MD[2, 17, 2, 0] = np.nextafter(run.MD[2, 17, 2, 0], np.float32(np.inf))
    elif what == "d mismatch":
        run.MD[2, 17, 1, 1] *= np.float32(1 + 1e-3)
    elif what == "alpha":
        run.MD[2, 5, 1, 2] = run.MD[2, 5, 1, 2] * np.float32(1 + 2.0 ** -18) + np.float32(2.0 ** -20)
    elif what in ("partial, tile", "RO, tile"):
        # 1% of the tile's sum of |products| for that row and channel: five
        # times the partial's bar (2^-9 of it); RO after tile 1 gets 1% of the
        # sum over tiles 0 and 1
        p = run.preps[1]
        vabs = np.abs(so.e4m3_decode(p.v_codes).astype(np.float64))
        pdec = so.e4m3_decode(run.P8[2, 9]).astype(np.float64)
        absdot = [float(pdec[j * 64:(j + 1) * 64] @ vabs[j * 64:(j + 1) * 64, 33]) for j in range(2)]
        if what == "partial, tile":
            run.PART[2, 9, 1, 33] += np.float32(0.01 * absdot[1] + 1.0)
        else:
            run.RO[2, 9, 1, 33] += np.float32(0.01 * (absdot[0] + absdot[1]) + 1.0)
    elif what == "reciprocal":
        run.R[2, 4] *= np.float32(1 + 1e-3)
    elif what == "capture O != fast O":
        run.Oc[0, 1, 5, 0] ^= 1
    elif what == "O entries beyond":
        o = so.bf16_bits_to_f32(run.O[0, 1, 5:6, 0:1])[0, 0] + np.float32(0.25)
        bits = (np.array([o], np.float32).view(np.uint32) >> 16).astype(np.uint16)
        run.O[0, 1, 5, 0] = run.Oc[0, 1, 5, 0] = bits[0]
    elif what == "masked P8 not zero":
        run.P8[0, 3, NKV + 2] = 0x38
    elif what == "P8 two codes":
        run.P8[0, 3, 10] = np.uint8(int(run.P8[0, 3, 10]) + 2)
    else:
        raise ValueError(what)
    return run


@pytest.mark.parametrize("what", ["k_mean", "q_scale", "k_scale", "v_scale", "q codes", "k codes", "v codes",
                                  "S mismatch", "m mismatch", "d mismatch", "alpha", "partial, tile",
                                  "RO, tile", "reciprocal", "capture O != fast O", "O entries beyond",
                                  "masked P8 not zero"])
def test_comparison_names_the_planted_stage(clean, what):
    run = _plant(clean, what)
    with pytest.raises(AssertionError) as e:
        _check_all(run)
    assert what in str(e.value), "planted %r, comparison said %r" % (what, str(e.value)[:200])


def test_comparison_rejects_a_probability_code_two_steps_off(clean):
    """P8 may differ by one code at a rounding near-tie, never by two."""
    run = _plant(clean, "P8 two codes")
    with pytest.raises(AssertionError) as e:
        _check_all(run)
    assert "P8 code off by 2" in str(e.value)
