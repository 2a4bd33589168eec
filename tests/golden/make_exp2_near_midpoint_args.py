"""Writes exp2_near_midpoint_args.txt: float32 arguments x in [-150, 0] whose
2^x lies closest to a midpoint between adjacent float32 values, the inputs on
which a float32 exp2 is hardest to round correctly.

Exhaustive scan of every float32 in [-150, 0] (about 1.1e9 values, about a
minute): 2^x in float64, distance to the nearest float32 midpoint in float32
units.  Only arguments are stored; the tests compute the expected values with
mpmath.  Usage: python tests/golden/make_exp2_near_midpoint_args.py
"""
import os

import numpy as np

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exp2_near_midpoint_args.txt")
KEEP = 200


def main():
    lo_bits = 0x80000000                                   # -0.0
    hi_bits = int(np.float32(-150.0).view(np.uint32))
    chunk = 1 << 24
    best = []
    for start in range(lo_bits, hi_bits + 1, chunk):
        b = np.arange(start, min(start + chunk, hi_bits + 1), dtype=np.uint64).astype(np.uint32)
        x = b.view(np.float32)
        with np.errstate(all="ignore"):
            y = np.exp2(x.astype(np.float64))
            r = y.astype(np.float32)
            lo = np.where(r.astype(np.float64) > y, np.nextafter(r, np.float32(-np.inf)), r)
            hi = np.nextafter(lo, np.float32(np.inf))
            lo64, hi64 = lo.astype(np.float64), hi.astype(np.float64)
            dist = np.abs(y - (lo64 + hi64) / 2) / (hi64 - lo64)
        sel = np.argsort(dist)[:KEEP]
        best.extend((float(dist[i]), int(b[i])) for i in sel)
        best = sorted(best)[:KEEP]
    with open(OUT, "w") as fh:
        fh.write("# float32 bit patterns of x in [-150, 0] with 2^x closest to a float32 rounding midpoint\n")
        fh.write("# (distance in float32 units, as evaluated in float64); written by make_exp2_near_midpoint_args.py\n")
        for d, bits in best:
            fh.write("%08x %.3e\n" % (bits, d))


if __name__ == "__main__":
    main()
