"""Every head and every row of a full-size workload against the oracle.

Not collected by pytest (the long video workload takes about four minutes of
oracle time on 16 cores); run it on a machine with the GPU:

    python tests/full_size_parity.py dit_block      # or long_video, headdim64, ...
    python tests/full_size_parity.py dit_block --summary PATH   # also append the summary line to PATH

The oracle runs first, one (b,h) per task in up to 16 spawned single-threaded
processes (before this process touches the GPU); then the library runs the
prep and the forward once.  Checked: K mean, every scale and every code of
every head bit-exact; the output per element within max(1e-2, one bf16 unit of
the oracle's value) and mean-rel <= 1e-3 over the whole tensor.  The units of
rows over that per-element bar are run again with checkpoint capture and
judged as the parity tests judge them, with the share of any FP8 probability
code that differs from the oracle's.
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


def _oracle_head(args):
    q, k, v = args
    from threadpoolctl import threadpool_limits

    from oracle import sage_oracle as so
    with threadpool_limits(limits=1):
        p = so.prep_bh(q, k, v)
        O = so.attention_rows(p)
    return p.k_mean, p.q_scale, p.k_scale, p.v_scale, p.q_codes, p.k_codes, p.v_codes, O


def main(workload: str, procs: int, summary_path: str | None = None) -> None:
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs

    w = WORKLOADS[workload]
    q, k, v = make_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    tasks = [(q[b, h].float().numpy(), k[b, h].float().numpy(), v[b, h].float().numpy()) for b, h in heads]
    t0 = time.time()
    ref = []
    with ProcessPoolExecutor(procs, mp_context=mp.get_context("spawn")) as ex:
        for i, r in enumerate(ex.map(_oracle_head, tasks)):
            ref.append(r)
            if (i + 1) % 8 == 0 or i + 1 == len(tasks):
                print("oracle: %d/%d heads (%.0f s)" % (i + 1, len(tasks), time.time() - t0), flush=True)

    from oracle import sage_oracle as so
    from tests import test_gpu_parity as tp

    nqb = -(-w.Nq // 128)
    run = tp.Run(q, k, v, [0])
    stats = tp.OStats()
    over_units, n_over = set(), 0
    for bh, (b, h) in enumerate(heads):
        km, qs, ks, vs, qc, kc, vc, O_ref = ref[bh]
        for name, got, want in (("k_mean", run.k_mean[bh], km), ("q_scale", run.q_scale[bh], qs),
                                ("k_scale", run.k_scale[bh], ks), ("v_scale", run.v_scale[bh], vs)):
            assert np.array_equal(tp._bits32(got), tp._bits32(want)), (name, bh)
        gq, gk, gv = run.codes(bh)
        assert np.array_equal(gq, qc) and np.array_equal(gk, kc) and np.array_equal(gv, vc), ("codes", bh)
        g = so.bf16_bits_to_f32(run.O[b, h]).astype(np.float64)
        r = so.bf16_bits_to_f32(O_ref).astype(np.float64)
        bad = np.abs(g - r) > np.maximum(tp.O_MAX_ABS, tp.bf16_ulp(r))
        n_over += int(bad.sum())
        over_units.update(bh * nqb + int(row) // 128 for row in np.unique(np.nonzero(bad)[0]))
        # entries over the bar are judged below, with capture; the rest here
        stats.add_o(run.O[b, h], O_ref, np.where(bad, np.inf, 0.0))
    mean_rel = stats.sum_abs_diff / stats.sum_abs_ref
    print("prep bit-exact on all %d heads; output: max_abs %.3g, mean_rel %.3g over %d entries (%d bit-equal), "
          "%d above 1e-2 within one bf16 unit (R20), %d entries in %d units over max(1e-2, 1 bf16 ulp)"
          % (len(heads), stats.max_abs, mean_rel, stats.n_o, stats.n_equal, stats.n_r20, n_over,
             len(over_units)), flush=True)
    assert mean_rel <= tp.O_MEAN_REL
    budget = tp.O_OVER_FRAC_GAUSSIAN if workload in ("single_tile", "dit_block", "long_video") else tp.O_OVER_FRAC
    assert stats.n_over <= budget * stats.n_o, "%d entries over 1e-2 (budget %g)" % (stats.n_over, budget)
    n_r21 = 0
    if over_units:
        units = sorted(over_units)
        again = tp.Run(q, k, v, units)
        preps = {u // nqb: again.oracle_prep(u // nqb) for u in units}
        st2 = tp.OStats()
        tp.check_units(again, st2, preps)
        st2.check(None)              # units chosen for their entries over the bar: no budget
        n_r21 = st2.n_r21
        assert n_r21 == n_over, "every entry over the per-element bar must lie within a flipped P8 code's share"
    summary = {"workload": workload, "heads": len(heads), "units": len(heads) * nqb, "entries": stats.n_o,
               "bit_equal": stats.n_equal, "max_abs": stats.max_abs, "mean_rel": mean_rel,
               "over_1e-2": stats.n_over, "pass_by_R20": stats.n_r20, "pass_by_R21": n_r21,
               "kernel_source_hash": kernel_source_hash()}
    if summary_path:
        os.makedirs(os.path.dirname(os.path.abspath(summary_path)), exist_ok=True)
        with open(summary_path, "a") as fh:
            fh.write(json.dumps(summary) + "\n")
    print("full-size parity: %s, %d heads, %d units: OK %s" % (workload, len(heads), len(heads) * nqb,
                                                              json.dumps(summary)), flush=True)


def kernel_source_hash() -> str:
    """The forward's source hash as bench.py computes it (comments and blank
    space removed), so a summary names the kernel it was taken on."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_for_hash", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.kernel_source_hash()


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("workload", nargs="?", default="dit_block")
    ap.add_argument("--summary", default=None, help="append the JSON summary line to this file")
    a = ap.parse_args()
    main(a.workload, int(os.environ.get("ORACLE_PROCS", min(16, len(os.sched_getaffinity(0))))), a.summary)
