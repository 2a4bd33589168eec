"""Tile indices past 65536 against the oracle: one head of 4.2M keys.

Not collected by pytest (about a minute of oracle time per head dimension,
over the suite's per-test limit); run on a machine with the GPU:

    python tests/long_key_parity.py 128      # or 64

The construction is the one of tests/test_gpu_accuracy.py: 65536 + 40 full
64-key tiles and a ragged one, the keys from two tiles before tile 65536
onward shifted along a direction shared with every query so that they carry
over 90% of each row's softmax weight (a tile read from a wrong address would
change the output completely), K rounded to multiples of 2^-12 so that its
column sums are exact in float64.  The library runs prep and forward once.
Checked against the oracle: K mean, every scale and every Q, K and V code
bit-exact; the output on every one of the 130 rows within max(1e-2, one bf16
unit) per element and mean-rel <= 1e-3.  With --summary PATH, appends the
summary line to PATH.
"""

from __future__ import annotations

import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402


def main(D: int, summary_path: str | None = None) -> None:
    import torch

    from oracle import sage_oracle as so
    from quantized_exact_attention_amd import sage
    from tests import test_gpu_parity as tp

    Nq, split = 130, 65536 * 64
    Nkv, hot0 = split + 64 * 40 + 23, split - 128
    g = torch.Generator().manual_seed(23 + D)
    c = (14.0 * D ** 0.5) ** 0.5
    u = torch.ones(D) / D ** 0.5
    q = (torch.randn(Nq, D, generator=g) + c * u).to(torch.bfloat16)
    k = torch.randn(Nkv, D, generator=g)
    k[hot0:] += c * u
    k = (torch.round(k * 4096) / 4096).to(torch.bfloat16)
    v = torch.randn(Nkv, D, generator=g).to(torch.bfloat16)
    print("long keys: Nq=%d Nkv=%d D=%d (tiles %d)" % (Nq, Nkv, D, -(-Nkv // 64)), flush=True)

    dev = torch.device("cuda:0")
    quant = sage.sage_quant_prep(q[None, None].to(dev), k[None, None].to(dev), v[None, None].to(dev))
    out = sage.sage_attn_fwd(quant)
    torch.cuda.synchronize()
    O = out[0, 0].view(torch.int16).cpu().numpy().view(np.uint16)

    class R:
        pass
    run = R()
    run.quant = quant
    run.B, run.H, run.D = 1, 1, D
    run.k_mean = quant.k_mean.cpu().numpy().reshape(1, D)
    run.q_scale = quant.q_scale.cpu().numpy().reshape(1, quant.nqb)
    run.k_scale = quant.k_scale.cpu().numpy().reshape(1, quant.T)
    run.v_scale = quant.v_scale.cpu().numpy().reshape(1, D)
    run._q_codes, run._k_codes, run._v_codes = quant.q_codes, quant.k_codes, quant.v_codes
    run.codes = lambda bh: tp.Run.codes(run, bh)
    del out
    t0 = time.time()
    p = so.prep_bh(q.float().numpy(), k.float().numpy(), v.float().numpy())
    print("oracle prep: %.0f s" % (time.time() - t0), flush=True)
    tp.check_prep_bh(run, 0, p)
    print("prep bit-exact: K mean, scales, %d Q, K and V codes each" % (p.k_codes.size), flush=True)
    del quant, run
    torch.cuda.empty_cache()
    t0 = time.time()
    rows = np.arange(Nq)
    O_ref = so.attention_rows(p, rows)
    print("oracle attention, %d rows: %.0f s" % (Nq, time.time() - t0), flush=True)
    stats = tp.OStats()
    stats.add_o(O, O_ref)
    stats.check()
    summary = {"D": D, "Nq": Nq, "Nkv": Nkv, "tiles": -(-Nkv // 64), "entries": stats.n_o, "bit_equal": stats.n_equal,
               "max_abs": stats.max_abs, "mean_rel": stats.sum_abs_diff / stats.sum_abs_ref,
               "over_1e-2": stats.n_over, "pass_by_R20": stats.n_r20}
    if summary_path:
        os.makedirs(os.path.dirname(os.path.abspath(summary_path)), exist_ok=True)
        with open(summary_path, "a") as fh:
            fh.write(json.dumps(summary) + "\n")
    print("long-key parity OK", json.dumps(summary), flush=True)


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("D", nargs="?", type=int, default=128)
    ap.add_argument("--summary", default=None, help="append the JSON summary line to this file")
    a = ap.parse_args()
    main(a.D, a.summary)
