#!/usr/bin/env python3
"""Benchmark: FP8 MLA split-KV decode on one MI355X.

One step = the whole hot path for one decode step of one MLA layer: saturating FP8
quantisation of the step's Q, split-KV partial attention over the FP8 KV cache, and the
log-sum-exp combine to bf16.  KV and Q are resident in HBM before timing starts.  The KV
cache is held in several identical copies that the steps rotate through, so that no step
finds its KV in the 256 MB Infinity Cache left behind by the previous one.

Prints one JSON line.  `value` is microseconds per decode step on the batch-1, 128K-context
workload; the batch-16 workload is reported alongside.  `roofline` is for the decode kernel
(HBM-bound at 1 query token per request): algorithmic bytes = KV bytes + Q bytes per launch,
divided by the kernel's average duration from HIP events on its stream.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b1_128k")
    ap.add_argument("--also", default="b16_128k", help="second workload reported alongside ('' = none)")
    ap.add_argument("--splits", type=int, default=0, help="0 = planner")
    ap.add_argument("--rows-per-group", type=int, default=0, help="0 = planner")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, --steps times (the "
                         "reference kernel that calibrates HBM byte counters), then exit")
    return ap.parse_args()


def copy_probe(mib, steps):
    """A plain device-to-device copy of known size: each launch reads and writes exactly
    mib MiB, which is what the profiler's FETCH_SIZE / WRITE_SIZE should report for it."""
    import torch
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": steps}), flush=True)


def run_workload(key, steps, warmup, splits, rows_per_group, min_bytes=512 << 20):
    import torch
    import fp8_mla_split_amd as mla
    from fp8_mla_split_amd.workload import materialize
    from synthetic import WORKLOADS, q_f32

    w = WORKLOADS[key]
    dw = materialize(w)
    B, Sq, H = w.batch, w.q_tokens, w.heads
    kv_bytes = dw.kv_tokens * 576
    copies = max(1, -(-min_bytes // max(kv_bytes, 1)) + 1) if kv_bytes < min_bytes else 1
    pools = [dw.kv_pool8] + [dw.kv_pool8.clone() for _ in range(copies - 1)]
    q32 = torch.from_numpy(q_f32(w)).cuda()
    q8 = torch.empty_like(q32, dtype=torch.uint8)
    plan = mla.splitkv_plan(B, Sq, H, dw.max_seq_len)
    S = splits or plan.num_splits
    r = rows_per_group or plan.rows_per_group
    po = torch.empty((B, S, Sq * H, 512), dtype=torch.float32, device="cuda")
    pl = torch.empty((B, S, Sq * H), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Sq, H), dtype=torch.float32, device="cuda")

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        mla.quantize_fp8_sat(q32, dw.q_scale, out=q8)
        if ev is not None:
            ev[1].record()
        mla.decode_splitkv(q8, pools[i % copies], dw.page_table, dw.seq_lens, dw.q_scale,
                           dw.kv_scale, w.softmax_scale, dw.max_seq_len, S, r, po, pl)
        if ev is not None:
            ev[2].record()
        mla.splitkv_combine(po, pl, Sq, H, out=out, out_lse=lse)
        if ev is not None:
            ev[3].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    q_us = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
    dec_us = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3
    comb_us = np.array([e[2].elapsed_time(e[3]) for e in evs]) * 1e3
    step_us = np.array([e[0].elapsed_time(e[3]) for e in evs]) * 1e3

    q_bytes = B * Sq * H * 576
    algo = kv_bytes + q_bytes
    flops = 2.0 * B * Sq * H * dw.kv_tokens * (576 + 512)  # QK^T + PV, algorithmic
    res = {
        "workload": w.name, "batch": B, "heads": H, "q_tokens": Sq,
        "context": int(dw.max_seq_len), "kv_tokens": dw.kv_tokens,
        "num_splits": S, "rows_per_group": r, "kv_copies": copies,
        "us_per_step": total_ms * 1e3 / steps,
        "step_us_p10_p50_p90": [float(np.percentile(step_us, p)) for p in (10, 50, 90)],
        "quantize_q_us": float(q_us.mean()), "decode_us": float(dec_us.mean()),
        "combine_us": float(comb_us.mean()),
        "decode_us_p50": float(np.median(dec_us)),
        "kv_bytes": kv_bytes, "algo_bytes_decode": algo,
        "decode_gbps": algo / (dec_us.mean() * 1e3),
        "step_kv_gbps": kv_bytes / (total_ms * 1e6 / steps),
        "decode_mfma_tflops_algorithmic": flops / (dec_us.mean() * 1e6),
        "partial_bytes": B * S * Sq * H * 513 * 4,
    }
    del pools, po, pl, dw
    torch.cuda.empty_cache()
    return res


def cpu_baseline(key, budget_s):
    """The oracle as it stands, one decode step at a time on the host cores, until about
    budget_s seconds of work are done (the sample is a count of whole steps)."""
    from oracle import attention_fp64, quantize_e4m3_sat
    from synthetic import WORKLOADS, kv_request_f32, page_layout, q_f32, seq_lens_for
    from oracle import per_tensor_scale

    w = WORKLOADS[key]
    lens = seq_lens_for(w)
    P, table, _ = page_layout(w, lens)
    q = q_f32(w)
    kv = kv_request_f32(w, 0, int(lens[0]))
    qs, ks = per_tensor_scale(q), per_tensor_scale(kv)
    pool = np.zeros((1, P, 576), np.uint8)
    pool[0, :int(lens[0])] = quantize_e4m3_sat(kv, ks)
    del kv
    n, t0 = 0, time.perf_counter()
    while True:
        q8 = quantize_e4m3_sat(q[:1], qs)                       # per-step Q prep
        attention_fp64(q8, qs, pool, ks, table[:1], lens[:1], P, w.softmax_scale)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 50:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info())
    except Exception:
        cores = len(os.sched_getaffinity(0))
    steps_per_request = w.batch  # the oracle handles requests one after another
    us = el / n * 1e6 * steps_per_request
    return {"value": us, "unit": "us/step", "cores": cores, "kind": "oracle",
            "sample": f"{n} full decode steps of request 0 of {w.name} (Q quantize + fp64 "
                      f"attention over all {int(lens[0])} positions and {w.heads} heads), "
                      f"{el:.1f} s of host time"}


def main():
    a = _parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              f"(multi-GPU sharding is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if a.copy_probe_mib:
        copy_probe(a.copy_probe_mib, a.steps)
        return
    t_wall = time.time()
    main_res = run_workload(a.workload, a.steps, a.warmup, a.splits, a.rows_per_group)
    print(f"[bench] {a.workload}: {main_res['us_per_step']:.2f} us/step "
          f"(decode {main_res['decode_us']:.2f} us, {main_res['decode_gbps']:.0f} GB/s)",
          file=sys.stderr, flush=True)
    also = None
    if a.also:
        also = run_workload(a.also, max(20, a.steps // 4), max(5, a.warmup // 4), 0, 0)
        print(f"[bench] {a.also}: {also['us_per_step']:.2f} us/step "
              f"(decode {also['decode_us']:.2f} us, {also['decode_gbps']:.0f} GB/s)",
              file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(a.workload, a.cpu_seconds)
    achieved = main_res["decode_gbps"]
    line = {
        "metric": "µs/decode step + achieved KV-read HBM GB/s (% of peak), 128K ctx batch 1/16",
        "value": round(main_res["us_per_step"], 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_res["us_per_step"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded N(0,1) Q/KV, per-tensor scales)",
        "config": {k: main_res[k] for k in ("workload", "batch", "heads", "q_tokens", "context",
                                            "num_splits", "rows_per_group", "kv_copies")},
        "kv_read_gbps_step": round(main_res["step_kv_gbps"], 1),
        "kv_read_pct_of_peak_step": round(100 * main_res["step_kv_gbps"] / HBM_PEAK_GBPS, 2),
        "breakdown_us": {k: round(main_res[k], 3) for k in ("quantize_q_us", "decode_us",
                                                            "combine_us")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None,
                     "kernel": "decode_kernel (mla_decode_splitkv)",
                     "algorithmic_bytes_per_launch": main_res["algo_bytes_decode"],
                     "mfma_tflops_algorithmic": round(main_res["decode_mfma_tflops_algorithmic"], 1),
                     "mfma_peak_tflops_fp8": FP8_PEAK_TFLOPS},
        "cpu_baseline": cpu,
        "also": None if also is None else {
            "workload": also["workload"], "us_per_step": round(also["us_per_step"], 3),
            "decode_us": round(also["decode_us"], 3),
            "decode_gbps": round(also["decode_gbps"], 1),
            "decode_frac_of_hbm_peak": round(also["decode_gbps"] / HBM_PEAK_GBPS, 4),
            "num_splits": also["num_splits"], "rows_per_group": also["rows_per_group"]},
        "detail": main_res,
        "wall_s": round(time.time() - t_wall, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
