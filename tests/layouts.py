"""Host-side views of the operand-ordered code buffers (layouts from include/sage_attn.h).

Test infrastructure: these only move bytes, so GPU codes can be compared with
the oracle's row-major codes.
"""

import numpy as np


def i8_rows(codes: np.ndarray, BH: int, rows_pad: int, D: int) -> np.ndarray:
    """INT8 32-row-group operand order -> row-major [BH, rows_pad, D]."""
    NS = D // 32
    G = rows_pad // 32
    a = np.asarray(codes).reshape(BH, G, NS, 2, 32, 16)      # [bh, g, s, half, l, e]
    return a.transpose(0, 1, 4, 2, 3, 5).reshape(BH, rows_pad, D)


def v_rows(codes: np.ndarray, BH: int, T: int, D: int) -> np.ndarray:
    """E4M3 PV-operand order -> row-major [BH, T*64, D]."""
    NS = D // 32
    a = np.asarray(codes).reshape(BH, T, NS, 2, 2, 32, 4, 4)  # [bh, t, c, h, g, l, r, q]
    # key = 32h + 8r + 4g + q, channel = 32c + l
    return a.transpose(0, 1, 3, 6, 4, 7, 2, 5).reshape(BH, T * 64, D)
