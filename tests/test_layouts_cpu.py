"""The host-side layout views used by the GPU tests, checked against a direct
element-by-element transcription of the layouts documented in the header."""

import numpy as np

from tests.layouts import i8_rows, v_rows


def test_i8_operand_layout_roundtrip():
    rng = np.random.default_rng(0)
    for D in (64, 128):
        rows = 128
        src = rng.integers(-127, 128, (rows, D)).astype(np.int8)
        buf = np.zeros(rows * D, np.int8)
        NS = D // 32
        for r in range(rows):
            for c in range(D):
                g, l = divmod(r, 32)
                s, rem = divmod(c, 32)
                half, e = divmod(rem, 16)
                lane = l + 32 * half
                buf[((g * NS + s) * 64 + lane) * 16 + e] = src[r, c]
        assert np.array_equal(i8_rows(buf, 1, rows, D)[0], src)


def test_v_operand_layout_roundtrip():
    rng = np.random.default_rng(1)
    for D in (64, 128):
        T = 2
        src = rng.integers(0, 126, (T * 64, D)).astype(np.uint8)
        buf = np.zeros(T * 64 * D, np.uint8)
        NS = D // 32
        for t in range(T):
            for blk in range(NS):
                for half in range(2):
                    for lane in range(64):
                        for e in range(16):
                            key = 32 * half + 8 * (e // 4) + 4 * (lane // 32) + e % 4
                            ch = 32 * blk + lane % 32
                            off = (((t * NS + blk) * 2 + half) * 64 + lane) * 16 + e
                            buf[off] = src[t * 64 + key, ch]
        assert np.array_equal(v_rows(buf, 1, T, D)[0], src)
