"""The forward's reading of INT8 scores as floats, checked exhaustively on the CPU.

The INT8 product K.Q^T accumulates on top of the bit pattern 0x3E22F983 (the
inline constant 1/(2 pi)); the kernel reads each int32 result as a float32,
subtracts 1/(2 pi) and multiplies by the per-tile factor scaled by 2^26.  For
every score the product can reach (|s| <= 127 * 127 * 128) the subtraction must
give s * 2^-26 exactly and the scaled factor must be exact, so that the exp2
argument fma(s * 2^-26, c * 2^26, b) rounds the same real number s * c + b as
fma(float(s), c, b).  This is host arithmetic only (no GPU, no oracle).
"""

import numpy as np

BIAS = 0x3E22F983
LIMIT = 127 * 127 * 128          # largest |score| at D = 128 (and twice the D = 64 one)


def _decode(s):
    biased = (np.int64(BIAS) + s).astype(np.int32)
    one_over_2pi = np.array([BIAS], dtype=np.int32).view(np.float32)[0]
    return biased.view(np.float32) - one_over_2pi          # float32 subtraction, as on the GPU


def test_bias_is_the_inline_constant_one_over_two_pi():
    f = np.array([BIAS], dtype=np.int32).view(np.float32)[0]
    assert f == np.float32(1.0 / (2.0 * np.pi))


def test_decoding_exact_for_every_reachable_score():
    s = np.arange(-LIMIT, LIMIT + 1, dtype=np.int64)
    dec = _decode(s)
    assert dec.dtype == np.float32
    assert np.array_equal(dec.astype(np.float64), s.astype(np.float64) * 2.0 ** -26)
    # the biased integers order like the scores (the row max is taken on them)
    biased = (np.int64(BIAS) + s).astype(np.int32)
    assert np.all(np.diff(biased.astype(np.int64)) == 1)


def test_range_margin_below_the_binade():
    # one step beyond the lower margin leaves the binade [1/8, 1/4): not exact there
    s = np.array([-(BIAS & 0x7FFFFF) - 1], dtype=np.int64)
    assert -s[0] - 1 > LIMIT
    assert _decode(s)[0].astype(np.float64) != s[0] * 2.0 ** -26


def test_scaled_factor_is_exact():
    rng = np.random.default_rng(0)
    # per-tile factors (q scale * k scale * sm_scale * log2 e) over a wide range
    c = (10.0 ** rng.uniform(-30, 2, 4096)).astype(np.float32)
    cu = c * np.float32(2.0 ** 26)
    assert np.array_equal(cu.astype(np.float64), c.astype(np.float64) * 2.0 ** 26)
    # products of decoded scores with the scaled factor equal those of the scores
    s = np.arange(-LIMIT, LIMIT + 1, 997, dtype=np.int64)
    dec = _decode(s)
    for ci in c[:16]:
        a = dec * (ci * np.float32(2.0 ** 26))
        b = s.astype(np.float32) * ci
        assert np.array_equal(a, b)
