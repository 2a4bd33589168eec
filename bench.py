"""Benchmark of the quantized attention hot path (prep + fused forward) on one GPU.

One step = sage_quant_prep + sage_attn_fwd over one batch of seeded synthetic
bf16 inputs already resident in HBM.  Prints ONE JSON line:
  value       effective TFLOPS = 4*B*H*Nq*Nkv*D / (ms_per_step) (whole step)
  roofline    the fused forward kernel against the dense INT8/FP8 matrix peak,
              timed with HIP events on the stream it is launched on
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  mfma_peak_measured  the matrix cores' sustained INT8 and FP8 rates on this
              device (a pure matrix-instruction stream), with the forward's
              rate against them
Default workload: the long video-token sequence (B=1, H=24, N=32760, D=128).
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense INT8 (POP/s) and FP8 (FLOP/s) peak, 5.0 P
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
# matrix-core throughput per clock for INT8 and FP8: 256 CUs x 4 SIMDs x 2048 ops
MFMA_OPS_PER_CLOCK = 256 * 4 * 2048


def kernel_source_hash() -> str:
    """Hash of the forward's source with comments and blank space removed, so
    that an edit to a comment does not detach the recorded counters."""
    import re
    h = hashlib.sha256()
    for f in ("sage_fwd.hip", "sage_common.h"):
        with open(os.path.join(ROOT, "quantized_exact_attention_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per forward launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def shader_clock_ghz(samples):
    """Average shader clock per compute unit between two clock samples
    ([2, n, 4]: counter, 100 MHz counter, XCD id, hardware id): each unit's
    counter delta over the 100 MHz delta; median, min and max over the units
    seen in both samples (the shader-clock counter is kept per unit; a unit is
    the XCD id with the CU, shader-array and shader-engine fields, bits 8-14,
    of the hardware id)."""
    import numpy as np
    first = {}
    for row in samples[0]:
        first.setdefault((int(row[2]), (int(row[3]) >> 8) & 0x7F), row)
    ghz = []
    for row in samples[1]:
        a = first.get((int(row[2]), (int(row[3]) >> 8) & 0x7F))
        if a is not None and row[1] > a[1]:
            ghz.append((int(row[0]) - int(a[0])) / (int(row[1]) - int(a[1])) * 0.1)
    if not ghz:
        return None
    return {"median": float(np.median(ghz)), "min": float(min(ghz)), "max": float(max(ghz)),
            "units": len(set((int(r[2]), (int(r[3]) >> 8) & 0x7F) for r in samples[1]))}


def valu_rates(words, mix):
    """Cycles per instruction that each SIMD retired for every active role of
    the vector-issue sample `mix` (words: [VALU_WORKGROUPS, 16, 3] int of
    rounds, cycles, result word): per SIMD, the role's waves' instructions per
    cycle are summed; median over the SIMDs of the device."""
    import numpy as np
    from quantized_exact_attention_amd import sage
    roles = sage.VALU_MIXES[mix]
    w = np.asarray(words, dtype=np.float64).reshape(-1, 16, 3)
    out = {}
    for r in sorted(set(roles) - {0}):
        per_simd = []
        for simd in range(4):
            waves = [simd + 4 * g for g in range(4) if roles[g] == r]
            ipc = sum(w[:, i, 0] * sage.VALU_ROUND_INSTRUCTIONS[r] / np.maximum(w[:, i, 1], 1.0) for i in waves)
            per_simd.append(ipc)
        ipc = np.concatenate(per_simd)
        out[{1: "fma", 2: "exp", 3: "matrix"}[r]] = float(np.median(1.0 / ipc))
    return out


def _oracle_blocks(args):
    """Worker: time the oracle's attention over the given 128-row Q blocks of
    one head (single-threaded numpy in its own process)."""
    prep, nq, blocks, budget_s = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import sage_oracle as so

    done, t_att = 0, 0.0
    with threadpool_limits(limits=1):
        # one untimed row first: the first calls in a fresh process pay for
        # imports and first-use costs, which would weigh on short samples
        so.attention_rows(prep, np.arange(1))
        for qb in blocks:
            if t_att >= budget_s:
                break
            rows = np.arange(qb * 128, min(nq, qb * 128 + 128))
            t0 = time.perf_counter()
            so.attention_rows(prep, rows)
            t_att += time.perf_counter() - t0
            done += 1
    return done, t_att


def cpu_baseline(w, q, k, v, budget_s: float, workers: int):
    """Time the oracle on a bounded sample and scale to effective TFLOPS.

    Sample: the prep of head (0,0) plus 128-row Q blocks of that head in a
    seeded random order, spread over `workers` processes (one thread each) for
    about `budget_s` seconds each; the full-workload time is extrapolated
    linearly (prep per head x B*H, attention per block x B*H*ceil(Nq/128)) and
    divided by the number of workers.
    """
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import sage_oracle as so

    with threadpool_limits(limits=1):
        qh, kh, vh = (t[0, 0].float().numpy() for t in (q, k, v))
        t0 = time.perf_counter()
        p = so.prep_bh(qh, kh, vh)
        t_prep = time.perf_counter() - t0
    nqb = -(-w.Nq // 128)
    order = [int(x) for x in np.random.default_rng(0).permutation(nqb)]
    workers = max(1, min(workers, nqb))
    chunks = [order[i::workers] for i in range(workers)]
    results = None
    if workers > 1:
        try:
            import multiprocessing as mp
            from concurrent.futures import ProcessPoolExecutor
            # spawned children import numpy and the oracle only; a child that
            # dies breaks the pool (an exception) rather than being respawned
            with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
                futs = [ex.submit(_oracle_blocks, (p, w.Nq, c, budget_s)) for c in chunks]
                results = [f.result(timeout=4 * budget_s + 120) for f in futs]
        except Exception as e:                  # fall back to one thread in this process
            print("bench: oracle worker pool failed (%s); timing one thread" % e, file=sys.stderr, flush=True)
            workers, chunks = 1, [order]
    if results is None:
        results = [_oracle_blocks((p, w.Nq, chunks[0], budget_s))]
    blocks = sum(r[0] for r in results)
    t_att = sum(r[1] for r in results)          # core-seconds
    BH = w.B * w.H
    t_core = t_prep * BH + (t_att / blocks) * BH * nqb
    t_total = t_core / workers
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {
        "value": w.flops / t_total / 1e12,
        "unit": "TFLOPS",
        "cores": workers,
        "kind": "oracle",
        "host": {"cpu_model": cpu_model, "cores_available": len(os.sched_getaffinity(0))},
        "sample": "prep of head (0,0) of %d heads (%.2f s) + %d of that head's %d 128-row Q blocks "
                  "(%.1f core-s over %d single-threaded processes); extrapolated linearly to %d heads x %d "
                  "blocks: %.0f core-s, %.1f s on %d cores" % (BH, t_prep, blocks, nqb, t_att, workers, BH, nqb,
                                                             t_core, t_total, workers),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20, or 100 for workloads under 1 TFLOP)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: 10, or 200 for workloads under 1 TFLOP, "
                         "whose steps are too short for 10 of them to bring the card to its steady clock)")
    ap.add_argument("--workload", default="long_video")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle attention to time per worker process")
    ap.add_argument("--cpu-workers", type=int, default=min(16, len(os.sched_getaffinity(0))),
                    help="single-threaded oracle processes (independent Q blocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a kernel of known "
                         "HBM traffic, used to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path runs on a single GPU (requested --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_exact_attention_amd import build as qbuild
    from quantized_exact_attention_amd import sage
    from quantized_exact_attention_amd.synth import WORKLOADS, make_inputs

    if not os.path.exists(qbuild.LIB_PATH):
        qbuild.build()
    w = WORKLOADS[args.workload]
    if args.steps is None:
        args.steps = 100 if w.flops < 1e12 else 20
    if args.warmup is None:
        args.warmup = 200 if w.flops < 1e12 else 10
    print("bench: generating %s inputs B=%d H=%d Nq=%d Nkv=%d D=%d" % (w.name, w.B, w.H, w.Nq, w.Nkv, w.D),
          file=sys.stderr, flush=True)
    q, k, v = make_inputs(w)
    cpu_base = None
    if not args.no_cpu_baseline:
        # before the first GPU call: the oracle's worker processes then start
        # from a parent that holds no GPU state
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu_base = cpu_baseline(w, q, k, v, args.cpu_budget, args.cpu_workers)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    quant = sage.sage_quant_prep(qd, kd, vd)
    out = sage.sage_attn_fwd(quant)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # everything the timed loop needs is set up before the warm-up, so that the
    # GPU goes from the last warm-up step into the timed ones with no idle time
    # in between (an idle card lowers its clock, and the first timed steps then
    # ran up to 20% slower while it ramped back)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    clk = torch.zeros(2, sage.CLOCK_SAMPLES, 4, dtype=torch.int64, device=dev)
    sage.sage_clock_sample(clk[0], stream)       # first launch (code-object load) stays out of the timing
    for _ in range(args.warmup):
        sage.sage_quant_prep(qd, kd, vd, out=quant)
        sage.sage_attn_fwd(quant, out=out)
    # the host submits a short step (the DiT block's 0.3 ms) only a little
    # faster than the GPU runs it, so a garbage-collection pause inside the
    # loop would leave the GPU idle; collect now and not during the loop
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sage.sage_clock_sample(clk[0], stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        sage.sage_quant_prep(qd, kd, vd, out=quant)
        ev[i][1].record(stream)
        sage.sage_attn_fwd(quant, out=out)
        ev[i][2].record(stream)
    sage.sage_clock_sample(clk[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    print("bench: timed %d steps after %d warm-up steps" % (args.steps, args.warmup), file=sys.stderr, flush=True)
    sclk = shader_clock_ghz(clk.cpu().numpy())
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    prep_ms = [e[0].elapsed_time(e[1]) for e in ev]
    fwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    ms_per_step = wall * 1e3 / args.steps
    fwd_avg = statistics.mean(fwd_ms)
    achieved = w.flops / (fwd_avg * 1e-3) / 1e12

    res = {
        "metric": "effective attention TFLOPS (4*B*H*Nq*Nkv*D/t) and % of INT8/FP8 MFMA peak",
        "value": w.flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nkv": w.Nkv, "D": w.D,
                   "causal": False, "seed": w.seed, "outlier_p": w.outlier_p,
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": 100.0 * (w.flops / (ms_per_step * 1e-3) / 1e12) / MFMA_PEAK_TFLOPS,
        "step_ms_p50": statistics.median(step_ms),
        "step_ms_cv": statistics.pstdev(step_ms) / statistics.mean(step_ms),
        "step_ms_p10": statistics.quantiles(step_ms, n=10)[0] if len(step_ms) > 1 else step_ms[0],
        "step_ms_p90": statistics.quantiles(step_ms, n=10)[-1] if len(step_ms) > 1 else step_ms[0],
        "step_ms_each": [round(x, 4) for x in step_ms],
        "prep_ms_p50": statistics.median(prep_ms),
        "fwd_ms_p50": statistics.median(fwd_ms),
        "fwd_tflops_p50": w.flops / (statistics.median(fwd_ms) * 1e-3) / 1e12,
        "roofline": {
            "kernel": "k_attn_fwd<%d,false>" % w.D,
            "bound": "mfma",
            "achieved": achieved,
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / MFMA_PEAK_TFLOPS,
            "traffic": measured_traffic(w.name),
        },
        # average shader clock over the timed steps (s_memtime against the
        # 100 MHz counter, sampled on the launch stream before and after), and
        # the forward's matrix-core busy fraction that follows from its
        # algorithmic matrix work, its average duration and that clock
        "sustained_sclk_ghz": sclk,
        "fwd_mfma_busy_derived": ((w.flops / MFMA_OPS_PER_CLOCK) / (fwd_avg * 1e-3 * sclk["median"] * 1e9)
                                  if sclk else None),
        "cpu_baseline": None,
    }
    # The prep (three launches) is an HBM-bound stream: bytes of its two-pass
    # schedule (bf16 Q read once and its INT8 codes written; bf16 K and V read
    # twice and their one-byte codes written) per p50 launch time.
    eq, ekv = w.B * w.H * w.Nq * w.D, w.B * w.H * w.Nkv * w.D
    prep_bytes = 3 * eq + 10 * ekv
    prep_gbs = prep_bytes / (statistics.median(prep_ms) * 1e-3) / 1e9
    res["prep_roofline"] = {"kernels": "k_prep_pass1, k_prep_finalize, k_prep_pass2", "bound": "hbm",
                            "achieved": prep_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": prep_gbs / HBM_PEAK_GBS, "bytes": prep_bytes}
    # SHA-256 of the forward's BF16 output bytes (deterministic across launches)
    res["output_sha256"] = hashlib.sha256(out.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
    # The single-pass prep entry (K and V read once), timed apart from the step.
    sp_ms = []
    for i in range(args.warmup + args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sage.sage_quant_prep(qd, kd, vd, out=quant, single_pass=True)
        b.record(stream)
        if i >= args.warmup:
            sp_ms.append((a, b))
    torch.cuda.synchronize()
    res["prep_single_pass_ms_p50"] = statistics.median(a.elapsed_time(b) for a, b in sp_ms)
    # status word of the last single-pass call: 0 unless a workgroup stopped
    # waiting for its head's statistics (its outputs would then be invalid)
    res["prep_single_pass_status"] = quant.single_pass_status()
    # The paired forward schedule (three Q blocks per workgroup share one K/V
    # stream; same output), timed apart from the step.
    pf_ms = []
    for i in range(args.warmup + args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sage.sage_attn_fwd(quant, out=out, paired=True)
        b.record(stream)
        if i >= args.warmup:
            pf_ms.append((a, b))
    torch.cuda.synchronize()
    res["fwd_paired_ms_p50"] = statistics.median(a.elapsed_time(b) for a, b in pf_ms)
    # The Q-quantizing pair (sage_quant_prep_kv + sage_attn_fwd_q: the Q codes
    # never pass through memory; bit-identical output), timed as a step apart
    # from the headline one.
    kv = sage.sage_quant_prep_kv(kd, vd)
    out_q = sage.sage_attn_fwd_q(qd, kv)
    torch.cuda.synchronize()
    fq = []
    for i in range(args.warmup + args.steps):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        sage.sage_quant_prep_kv(kd, vd, out=kv)
        b.record(stream)
        sage.sage_attn_fwd_q(qd, kv, out=out_q)
        c.record(stream)
        if i >= args.warmup:
            fq.append((a, b, c))
    torch.cuda.synchronize()
    fq_step = statistics.median(a.elapsed_time(c) for a, b, c in fq)
    res["q_quantizing_pair"] = {
        "step_ms_p50": fq_step,
        "tflops_p50": w.flops / (fq_step * 1e-3) / 1e12,
        "prep_kv_ms_p50": statistics.median(a.elapsed_time(b) for a, b, c in fq),
        "fwd_q_ms_p50": statistics.median(b.elapsed_time(c) for a, b, c in fq),
        "output_equal": bool(torch.equal(out_q.view(torch.int16), out.view(torch.int16))),
    }
    del kv, out_q
    # The matrix cores' sustained rate on this device: a pure matrix-instruction
    # stream on every SIMD (INT8 32x32x32, then FP8 32x32x64), median of three
    # timed launches after a warm one, with the shader clock over them; the
    # forward's rate against it (half of its operations are INT8, half FP8).
    peak_dst = torch.empty(sage.PEAK_WORKGROUPS * 256, dtype=torch.int32, device=dev)
    peak = {}
    for kind, name in ((0, "int8"), (1, "fp8")):
        sage.sage_mfma_peak_sample(kind, 1, peak_dst, stream)
        torch.cuda.synchronize()
        rates = []
        sage.sage_clock_sample(clk[0], stream)
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            ops = sage.sage_mfma_peak_sample(kind, 4096, peak_dst, stream)
            b.record(stream)
            rates.append((a, b, ops))
        sage.sage_clock_sample(clk[1], stream)
        torch.cuda.synchronize()
        peak[name + "_tops"] = statistics.median(ops / (a.elapsed_time(b) * 1e-3) / 1e12 for a, b, ops in rates)
        sc = shader_clock_ghz(clk.cpu().numpy())
        peak[name + "_sclk_ghz"] = sc["median"] if sc else None
    peak["unit"] = "TOP/s"
    peak["fwd_frac_of_measured"] = achieved / (0.5 * (peak["int8_tops"] + peak["fp8_tops"]))
    res["mfma_peak_measured"] = peak
    # Vector issue rates on this device (cycles per wave64 instruction per
    # SIMD): FP32 FMA from one, three and four waves, exp from three waves, and
    # both beside a matrix-instruction stream on the same SIMD; the inputs of
    # the forward's per-wave-tile cycle account
    vdst = torch.empty(3 * 16 * sage.VALU_WORKGROUPS, dtype=torch.int32, device=dev)
    sage.sage_valu_sample(0, 1, vdst, stream)
    torch.cuda.synchronize()
    vr = {}
    for mix, name in ((0, "fma_1wave"), (1, "fma_3waves"), (2, "fma_4waves"), (3, "exp_3waves"),
                      (4, "fma_3waves_beside_matrix"), (5, "exp_3waves_beside_matrix")):
        sage.sage_valu_sample(mix, 200, vdst, stream)
        torch.cuda.synchronize()
        r = valu_rates(vdst.view(sage.VALU_WORKGROUPS, 16, 3).cpu().numpy(), mix)
        vr[name] = r["exp" if "exp" in name else "fma"]
        if "matrix" in r:                        # the matrix stream's own rate beside that work
            vr["matrix_beside_" + name.split("_")[0]] = r["matrix"]
    vr["unit"] = "shader-clock cycles per instruction per SIMD"
    res["valu_rates_measured"] = vr
    if w.name == "single_tile":
        # the pages quote this fixture's forward both batched and as single
        # launches (2,000 samples); time single launches the same way: one
        # forward, then a full synchronization, per sample
        single = []
        for _ in range(2000):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sage.sage_attn_fwd(quant, out=out)
            b.record(stream)
            torch.cuda.synchronize()
            single.append(a.elapsed_time(b))
        res["fwd_single_launch"] = {"samples": len(single), "p50_ms": statistics.median(single),
                                    "cv": statistics.pstdev(single) / statistics.mean(single)}
        # and back to back: 20 batches of 100 forwards with no synchronization
        # inside a batch, events around each batch; time per forward
        batches = []
        for _ in range(20):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(100):
                sage.sage_attn_fwd(quant, out=out)
            b.record(stream)
            torch.cuda.synchronize()
            batches.append(a.elapsed_time(b) / 100)
        res["fwd_back_to_back"] = {"batches": len(batches), "launches_per_batch": 100,
                                   "p50_ms": statistics.median(batches),
                                   "cv": statistics.pstdev(batches) / statistics.mean(batches)}
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["calibration_copy_bytes"] = n
    res["cpu_baseline"] = cpu_base
    print(json.dumps(res))


if __name__ == "__main__":
    main()
