"""Benchmark of the striped paged-attention hot path on one MI355X.

One step = every stripe's partial over all P stripes (plus cp_own_token_attn for the mixed workload) and the exact
merge of the partials, over one batch whose inputs are already resident in HBM. Without an own-token partial the step
is one cp_paged_attn_merged call (on the bf16 decode path: the persistent partial kernel and one kernel that finishes
split pieces and merges the stripes; elsewhere the partial and merge calls back to back); with one it is
cp_paged_attn_partial, cp_own_token_attn and cp_lse_merge. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b] [--no-cpu-baseline] [--no-other-configs]

The default workload is the Llama-3-8B-shaped GQA decode (32 q heads, 8 kv heads, head dim 128, page 16, P = 4
stripes, batch 64, context lengths uniform in [1024, 8192], bf16 with fp32 accumulation). `value` is KV GB/s:
algorithmic KV bytes (every context token's K and V read once) per second of wall-clock step time.

`value` and `ms_per_step` come from K back-to-back steps with nothing else enqueued between them. `roofline`
describes the dominant kernel (the partial call; with the merged call, its two kernels): algorithmic bytes per launch
over its average duration, measured with HIP events on the stream it runs on during K further steps (timing events
between the calls add ~10 us a step, so they are kept out of the step-time loop), against the 8 TB/s HBM peak (above
the ridge point: algorithmic flops against the 2.5 PFLOP/s bf16 MFMA peak). `traffic` is the measured HBM traffic per
launch from rocprofv3 counters, scaled by the counter/bytes ratio of a plain copy kernel (see ``--copy-calibration``
and the profiles directory); it is only filled in when the counters were taken on the current kernel build.

`cold_cache` times K further steps after an untimed 512 MiB write each, which evicts the 256 MB last-level cache: with
HIP events around every step (median, 10th and 90th percentiles), and without per-step events (`loop_ms`: events
around K write + step pairs, minus events around K writes alone, over K). `achievable` is the read rate of a plain
sequential 2 GiB stream (the library's streaming-read kernel, nontemporal loads) on the same device, and the step's
and the partial's KV rates as fractions of it.

`cpu_baseline` is the float64 CPU oracle timed on host cores over a bounded sample of the same workload.

`other_configs` (default llama8b run only): the tiny, long-context, MLA and mixed workloads timed the same way on the
same device after the headline (step rate, query tokens/s, the partial's roofline), so every workload's throughput is
on record; they are not the headline.

Warm-up is at least W steps and at least ``--min-warmup-s`` seconds of steps: the GPU's clocks settle only under
sustained load. Measured on the MLA workload, the partial takes ~560 us right after a few steps or after an idle
second and ~460 us after two seconds of back-to-back steps; the HBM-bound GQA decode changes by ~1%.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

# Counter-derived HBM traffic per partial launch for the default workload, from the rocprofv3 PMC runs recorded in
# profiles/ (FETCH_SIZE and WRITE_SIZE, scaled by the copy-kernel factor). Keyed by the kernel source hash it was
# taken on; ignored (traffic = null) when the kernel source has changed since.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_llama8b.json")


# Sources the GQA decode kernels are built from: the traffic record stays valid while none of them changes.
DECODE_SOURCES = ("cp_slot_map_amd/csrc/paged_decode.hip", "cp_slot_map_amd/csrc/common.h",
                  "cp_slot_map_amd/csrc/launch.h", "include/cpattn.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(os.path.basename(rel).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--min-warmup-s", type=float, default=2.0,
                    help="keep running untimed warm-up steps until this many seconds have passed (clock settling)")
    ap.add_argument("--workload", default="llama8b", choices=["tiny", "llama8b", "longctx", "mla", "mixed"])
    ap.add_argument("--interleave", type=int, default=1,
                    help="KV-cache interleave size of the pool (runs of that many slots per partner; 1 = plain rule)")
    ap.add_argument("--kv-dtype", default="same", choices=["same", "fp8"],
                    help="pool element type: the workload's dtype, or fp8 E4M3 codes with per-tensor descales")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time only the chosen workload (by default the llama8b run also times tiny, longctx, mla and "
                         "mixed and reports them under other_configs)")
    ap.add_argument("--other-warmup-s", type=float, default=1.0, help="warm-up seconds of each other workload")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU budget of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for the counter scale factor) and exit")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def stream_read_rate(nbytes=2 << 30, launches=20):
    """Read bandwidth (GB/s, median over launches) of the library's plain streaming-read kernel on this device: the
    achievable denominator next to the nominal HBM peak."""
    import numpy as np
    import torch

    from cp_slot_map_amd import api
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(16384, dtype=torch.int32, device="cuda")
    for _ in range(3):
        api.debug_stream_read(buf, sink=sink)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(launches)]
    for e0, e1 in ev:
        e0.record()
        api.debug_stream_read(buf, sink=sink)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(wl, budget_s):
    """Time the float64 oracle (stripe partials + exact merge per row) on a bounded sample of the workload's rows."""
    import numpy as np
    import torch

    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        blas_threads = max([p.get("num_threads", 1) for p in info] or [1])
        blas_lib = ",".join(sorted({str(p.get("internal_api", p.get("prefix", "?"))) for p in info})) or "?"
    except Exception:
        blas_threads, blas_lib = 1, "?"
    order = list(np.argsort(wl.ctx_len))
    rows = [order[0], order[-1]] + [b for b in np.random.default_rng(0).permutation(wl.batch).tolist()
                                    if b not in (order[0], order[-1])]
    spent, kv_bytes, tokens, done = 0.0, 0, 0, []
    per_token = wl.kv_bytes() / max(1, int(wl.ctx_len.astype(np.int64).sum()))
    # Rows in that order, over again from the start when the whole batch takes less than the budget (a steadier
    # figure); the budget is checked after each row.
    passes = max(1, min(50, int(budget_s / 0.5)))
    for b in rows * passes:
        rv = workloads.row_values(wl, int(b), "cuda")
        q, k, v = rv.q.cpu(), rv.k_ctx.cpu(), rv.v_ctx.cpu()
        if wl.kv_dtype == "fp8":
            k = oracle.dequantize_e4m3(k.view(torch.uint8), wl.k_descale)
            v = oracle.dequantize_e4m3(v.view(torch.uint8), wl.v_descale)
        kn = rv.k_new.cpu() if rv.k_new is not None else None
        vn = rv.v_new.cpu() if rv.v_new is not None else None
        del rv
        t0 = time.perf_counter()
        oracle.row_partials(q, k, v, wl.partners, wl.scale, kn, vn, interleave=wl.interleave)
        spent += time.perf_counter() - t0
        kv_bytes += int(wl.ctx_len[b]) * per_token
        tokens += int(wl.new_len[b])
        done.append(int(b))
        if spent >= budget_s:
            break
    torch.cuda.synchronize()
    return {
        "value": round(kv_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": f"{len(done)} row evaluations over {len(set(done))} of {wl.batch} rows (shortest and longest "
                  f"included; {len(done) / wl.batch:.1f} passes over the batch), {int(kv_bytes / per_token)} context "
                  f"tokens, float64 numpy on {blas_lib} with {blas_threads} threads, {spent:.1f} s; query tokens/s "
                  f"{tokens / spent:.2f}",
        "query_tokens_per_s": round(tokens / spent, 3),
    }


KERNEL_NAMES = {
    "llama8b": "cp_paged_attn_merged (gqa_decode_persist_kernel + gqa_decode_finish_kernel)",
    "longctx": "cp_paged_attn_merged (gqa_decode_persist_kernel + gqa_decode_finish_kernel)",
    "mla": "cp_paged_attn_partial (mla_plan_kernel + mla_decode_kernel)",
    "mixed": "cp_paged_attn_partial + cp_own_token_attn (gqa_extend_kernel, context and own-token)",
    "tiny": "cp_paged_attn_partial (paged_generic_kernel)",
}


def measure(wl, K, warmup, min_warmup_s, cold=True, achievable_gbs=None):
    """Time the hot-path step of workload ``wl`` (inputs resident in HBM): step rate from K back-to-back steps, the
    partial call's duration from HIP events on its stream during K more steps, and (``cold``) the step after a 512 MiB
    write that evicts the last-level cache. Returns a dict of figures."""
    import numpy as np
    import torch

    from cp_slot_map_amd import pool

    batch = pool.build_batch(wl, "cuda", fill=0.0)
    plan = pool.StepPlan(batch, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()

    t_warm = time.perf_counter()
    warm_steps = 0
    while warm_steps < warmup or time.perf_counter() - t_warm < min_warmup_s:
        for _ in range(10 if warm_steps >= warmup else 1):
            plan.run()
            warm_steps += 1
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_warm

    # Step time: K back-to-back steps with nothing else on the stream (events between the calls cost ~10 us a step).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        plan.run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Kernel durations: K more steps with HIP events around the partial (with the fused plan: the merged call) and the
    # merge, recorded on the stream the calls run on (the plan launches on torch's current stream).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        plan.partial()
        plan.own_token()
        ev[i][1].record()
        plan.combine()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    part_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    merge_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    res = {"wall": wall, "warm_steps": warm_steps, "warm_s": warm_s, "part_ms": part_ms, "merge_ms": merge_ms,
           "wall_ev": wall_ev, "fused": plan.fused}
    if cold:
        # Cold caches. (a) K steps, each after an untimed 512 MiB write that evicts the 256 MB last-level cache, timed
        # with HIP events around the step: median and 10th / 90th percentiles. (b) Without per-step events: two events
        # around K (write + step) pairs and two around K writes alone; the difference over K is the step.
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            scratch.fill_(i & 0xFF)
            cold_ev[i][0].record()
            plan.run()
            cold_ev[i][1].record()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        for i in range(K):
            scratch.fill_(i & 0xFF)
            plan.run()
        e[1].record()
        e[2].record()
        for i in range(K):
            scratch.fill_(i & 0xFF)
        e[3].record()
        torch.cuda.synchronize()
        res["cold_ms"] = np.array([cold_ev[i][0].elapsed_time(cold_ev[i][1]) for i in range(K)])
        res["cold_loop_ms"] = (e[0].elapsed_time(e[1]) - e[2].elapsed_time(e[3])) / K
        del scratch
    del plan, batch
    torch.cuda.empty_cache()
    return res


def summarize(wl, m, traffic=None):
    """Rates and the roofline of one workload's measurement."""
    import numpy as np

    K = len(m["part_ms"])
    ms_per_step = m["wall"] * 1e3 / K
    kv_bytes = wl.kv_bytes()
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    part_avg = float(np.mean(m["part_ms"]))
    achieved = kv_bytes / (part_avg * 1e-3) / 1e9
    # Algorithmic flops of the timed calls: every (query token, context token) pair costs Hq * 2 * (D + Dv), and so does
    # every (query token, visible in-step key) pair of the own-token call when the step has one (n (n + 1) / 2 a row).
    pairs = float(wl.ctx_len.astype(np.int64) @ wl.new_len.astype(np.int64))
    if wl.own_token:
        n = wl.new_len.astype(np.int64)
        pairs += float((n * (n + 1) // 2).sum())
    flops = pairs * wl.num_q_heads * 2 * (wl.head_dim + wl.head_dim_v)
    kernel = KERNEL_NAMES.get(wl.name, "cp_paged_attn_partial")
    if wl.kind == "mla" and wl.kv_dtype == "fp8":
        kernel = "cp_paged_attn_partial (mla_plan_kernel + mla_decode_kernel over the fp8 latent pool)"
    # The roofline that bounds the partial: HBM below the ridge point (peak flops / peak bytes), MFMA above it.
    mfma_bound = flops / kv_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) if kv_bytes else False
    tf = flops / (part_avg * 1e-3) / 1e12
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": kernel,
                "flops_per_launch": flops, "hbm_achieved_GBs": round(achieved, 2)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                "bytes_per_launch": kv_bytes}
    out = {"value": round(value, 2), "ms_per_step": round(ms_per_step, 5), "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
           "query_tokens_per_s": round(wl.num_tokens / (ms_per_step * 1e-3), 1),
           "kernel_ms": {"partial_avg": round(part_avg, 5), "partial_min": round(float(np.min(m["part_ms"])), 5),
                         "merge_avg": round(float(np.mean(m["merge_ms"])), 5),
                         "step_with_events": round(m["wall_ev"] * 1e3 / K, 5)},
           "roofline": roof, "tflops_partial": round(tf, 3), "mfma_frac_partial": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    if "cold_ms" in m:
        c = m["cold_ms"]
        out["cold_cache"] = {"median_ms": round(float(np.median(c)), 5), "p10_ms": round(float(np.percentile(c, 10)), 5),
                             "p90_ms": round(float(np.percentile(c, 90)), 5),
                             "GBs_at_median": round(kv_bytes / (float(np.median(c)) * 1e-3) / 1e9, 2),
                             "loop_ms": round(m["cold_loop_ms"], 5),
                             "GBs_loop": round(kv_bytes / (m["cold_loop_ms"] * 1e-3) / 1e9, 2)}
    return out, value, achieved


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the whole striped path runs on a single MI355X "
              f"(all P stripes resident); --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads

    if args.copy_calibration:
        copy_calibration()
        return
    torch.cuda.set_device(0)
    wl = workloads.make(args.workload, interleave=args.interleave, kv_dtype=args.kv_dtype)
    K = args.steps
    m = measure(wl, K, args.warmup, args.min_warmup_s)
    read_gbs = stream_read_rate()

    traffic = None
    if os.path.exists(TRAFFIC_RECORD):
        rec = json.load(open(TRAFFIC_RECORD))
        if rec.get("kernel_hash") == kernel_source_hash() and rec.get("workload") == wl.name:
            traffic = rec.get("bytes_per_launch")
    head, value, achieved = summarize(wl, m, traffic)
    kv_bytes = wl.kv_bytes()
    result = {
        "metric": "striped paged-attention decode: KV GB/s (% of HBM peak) and query tokens/s",
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_run": {"steps": m["warm_steps"], "seconds": round(m["warm_s"], 2)},
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "page_size": wl.page_size, "partners": wl.partners,
                   "ctx_tokens": int(wl.ctx_len.astype(np.int64).sum()), "query_tokens": wl.num_tokens,
                   "seed": wl.seed, "kv_bytes": kv_bytes, "interleave": wl.interleave, "kv_dtype": wl.kv_dtype},
        "hbm_frac_step": head["hbm_frac_step"],
        "query_tokens_per_s": head["query_tokens_per_s"],
        "kernel_ms": head["kernel_ms"],
        "roofline": head["roofline"],
        "cold_cache": head["cold_cache"],
        "achievable": {"kernel": "stream_read_kernel (cp_debug_stream_read, 2 GiB sequential read)",
                       "read_GBs": round(read_gbs, 2), "value_frac": round(value / read_gbs, 4),
                       "partial_frac": round(achieved / read_gbs, 4)},
        "tflops_partial": head["tflops_partial"],
        "mfma_frac_partial": head["mfma_frac_partial"],
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    # The other workloads, on the same clock (not the headline): step rate, tokens/s and the partial's roofline.
    if not args.no_other_configs and args.workload == "llama8b" and args.interleave == 1 and args.kv_dtype == "same":
        others = {}
        for name in ("tiny", "longctx", "mla", "mixed"):
            owl = workloads.make(name)
            om = measure(owl, min(K, 20), 3, args.other_warmup_s, cold=False)
            o, _, _ = summarize(owl, om)
            r = o["roofline"]
            others[name] = {"GBs": o["value"], "ms_per_step": o["ms_per_step"], "hbm_frac_step": o["hbm_frac_step"],
                            "query_tokens_per_s": o["query_tokens_per_s"], "partial_ms": o["kernel_ms"]["partial_avg"],
                            "roofline": {k: r[k] for k in ("bound", "achieved", "unit", "frac", "kernel")},
                            "mfma_frac_partial": o["mfma_frac_partial"], "kv_bytes": owl.kv_bytes(),
                            "query_tokens": owl.num_tokens}
        result["other_configs"] = others
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
