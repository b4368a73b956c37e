#!/usr/bin/env python3
"""Benchmark: FP8 MLA split-KV decode on one MI355X.

One step = the whole hot path for one decode step of one MLA layer: saturating FP8
quantisation of the step's Q (fp32 -> e4m3), split-KV partial attention over the FP8 KV
cache, and the log-sum-exp combine to bf16.  Q (fp32) and the FP8 KV cache are resident in
HBM before timing starts.  The KV cache is held in several identical copies that consecutive
steps rotate through (at least 512 MiB in total), so that no step finds its KV in the
256 MiB Infinity Cache left behind by the previous one.

The timed steps are captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed, so
host launch overhead is not part of the measurement; the region is bracketed by a device
synchronisation and HIP events on the launch stream.  The decode kernel's own duration for
the roofline comes from a second graph that holds only decode launches, timed the same way.

Prints one JSON line.  `value` is microseconds per decode step on the batch-1, 128K-context
workload; the batch-16 workload is reported alongside.  `roofline` is for the decode kernel
(HBM-bound at one query token per request): algorithmic bytes = KV bytes + Q bytes per
launch (576 B per cached token, 576 B per query row), divided by its average duration.
`extras` (skipped with --no-extras) holds reference rates measured in the same run (a
streaming HBM read, a device copy, KV-sized quantisation), p10/p50/p90 of single timed
steps, and decode + combine time over a sweep of split counts beside the planner's choice.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "µs/decode step + achieved KV-read HBM GB/s (% of peak), 128K ctx batch 1/16"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b1_128k")
    ap.add_argument("--also", default="b16_128k",
                    help="second workload reported alongside ('' = none)")
    ap.add_argument("--splits", type=int, default=0, help="0 = planner")
    ap.add_argument("--order", choices=("request", "longest"), default="request",
                    help="dispatch order of the requests' workgroups (longest first balances "
                         "mixed lengths)")
    ap.add_argument("--q-lens", default="",
                    help="comma-separated query-token count per request (verify step with a "
                         "different number of draft tokens per request); empty = all q_tokens")
    ap.add_argument("--rows-per-group", type=int, default=0, help="0 = planner")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python instead of replaying graphs "
                         "(what a profiler run needs to see individual launches clearly)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the HBM probes, per-step percentiles and the split sweep")
    ap.add_argument("--prep-only", action="store_true",
                    help="time only the cache-preparation entry points (KV append, quantise "
                         "with a device-derived scale) and print their JSON")
    ap.add_argument("--cp-workload", default="",
                    help="time only one GPU's share of a context-parallel decode of this "
                         "workload over 8 GPUs and print its JSON")
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


def _time_graph(g, reps):
    """Average milliseconds of one replay of g over reps replays (HIP events on the stream
    the graph is launched on)."""
    import torch
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


WARM_MS, BLOCK_MS, BLOCKS = 100.0, 40.0, 5


def _time_graph_steady(g):
    """Milliseconds of one replay of g in steady state: replays for at least WARM_MS of GPU
    time first (clocks and caches settle), then BLOCKS timed blocks of at least BLOCK_MS each;
    the median of the blocks' per-replay averages, and the number of replays timed."""
    one = _time_graph(g, 1)
    n_warm = max(2, int(WARM_MS / max(one, 1e-3)) + 1)
    one = _time_graph(g, n_warm)
    n = max(2, int(BLOCK_MS / max(one, 1e-3)) + 1)
    blocks = [_time_graph(g, n) for _ in range(BLOCKS)]
    return float(np.median(blocks)), n * BLOCKS


def run_workload(key, steps, warmup, splits, rows_per_group, eager=False, min_bytes=512 << 20,
                 dev_scales=False, q_lens=None, longest_first=False):
    """One decode step = Q quantise + split-KV decode + combine, timed over `steps` steps.
    dev_scales: Q's scale is derived on the device (mla_quantize_fp8_sat_dynamic) and the
    decode and combine read both scales from device memory."""
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
    plan = mla.splitkv_plan(B, Sq, H, dw.max_seq_len, total_kv_tokens=dw.kv_tokens)
    S = splits or plan.num_splits
    r = rows_per_group or plan.rows_per_group
    po = torch.empty((B, S, Sq * H, 512), dtype=torch.float16, device="cuda")
    pl = torch.empty((B, S, Sq * H), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Sq, H), dtype=torch.float32, device="cuda")

    qs_dev = torch.empty(1, dtype=torch.float32, device="cuda")
    ks_dev = torch.tensor([dw.kv_scale], dtype=torch.float32, device="cuda")
    ws = torch.empty(mla.QUANTIZE_DYNAMIC_WORKSPACE_BYTES // 4, dtype=torch.int32, device="cuda")
    q_scale = qs_dev if dev_scales else dw.q_scale
    kv_scale = ks_dev if dev_scales else dw.kv_scale

    def quantize():
        if dev_scales:
            mla.quantize_fp8_sat_dynamic(q32, out=q8, scale=qs_dev, workspace=ws)
        else:
            mla.quantize_fp8_sat(q32, dw.q_scale, out=q8)

    ql = None
    if q_lens:
        if len(q_lens) != B:
            raise SystemExit(f"--q-lens needs {B} counts for {w.name}")
        ql = torch.tensor(q_lens, dtype=torch.int32, device="cuda")

    order = None
    if longest_first:  # the caller knows the lengths: longest requests dispatched first
        order = torch.from_numpy(np.argsort(-dw.seq_lens_host, kind="stable")
                                 .astype(np.int32)).cuda()

    def decode(i):
        mla.decode_splitkv(q8, pools[i % copies], dw.page_table, dw.seq_lens, q_scale,
                           kv_scale, w.softmax_scale, dw.max_seq_len, S, r, po, pl, q_lens=ql,
                           order=order)

    def combine():
        mla.splitkv_combine(po, pl, Sq, H, kv_scale, out=out, out_lse=lse)

    def step(i):
        quantize()
        decode(i)
        combine()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    res = {"workload": w.name, "batch": B, "heads": H, "q_tokens": Sq,
           "context": int(dw.max_seq_len), "kv_tokens": dw.kv_tokens, "num_splits": S,
           "rows_per_group": r, "kv_copies": copies, "timing": "eager" if eager else "hip_graph",
           "scales": "device (Q amax on the GPU)" if dev_scales else "host"}
    if q_lens:
        res["q_lens"] = list(q_lens)
    if longest_first:
        res["order"] = "longest first"
    if eager:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            evs[i][0].record()
            quantize()
            evs[i][1].record()
            decode(i)
            evs[i][2].record()
            combine()
            evs[i][3].record()
        t1.record()
        torch.cuda.synchronize()
        step_us = t0.elapsed_time(t1) * 1e3 / steps
        q_us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
        dec_us = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3
        comb_us = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) * 1e3
    else:
        # a graph holds a whole number of rotations over the KV copies, so that replays
        # back to back still find each copy `copies` steps after its last use
        gsteps = -(-steps // copies) * copies
        stream = torch.cuda.Stream()
        graphs = {}
        for name, fn in (("step", step), ("quantize", lambda i: quantize()), ("decode", decode),
                         ("combine", lambda i: combine())):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(gsteps):
                    fn(i)
            graphs[name] = g
        torch.cuda.synchronize()
        timed = {}
        for name, g in graphs.items():
            ms, reps = _time_graph_steady(g)
            timed[name] = ms * 1e3 / gsteps
            if name == "step":
                res["graph_steps"], res["timed_steps"] = gsteps, gsteps * reps
        step_us, q_us = timed["step"], timed["quantize"]
        dec_us, comb_us = timed["decode"], timed["combine"]
        del graphs

    q_bytes = B * Sq * H * 576
    algo = kv_bytes + q_bytes
    # QK^T + PV, algorithmic: 2 * 1088 flops per (query row, cached token) of each request
    # (kv_tokens already sums the requests' lengths); the kernel executes 50 FP8 MFMAs of
    # 32x32x64 per 32 rows x 64 tokens (P.V twice, hi and lo): 3200 flops per (row, token)
    # with per-request counts only the present query rows count as algorithmic work (the
    # kernel skips row groups that hold no present row)
    row_tokens = Sq * dw.kv_tokens if not q_lens else float(np.dot(
        np.clip(np.asarray(q_lens), 0, Sq), dw.seq_lens_host.astype(np.float64)))
    flops = 2.0 * H * row_tokens * (576 + 512)
    flops_exec = 3200.0 * H * row_tokens
    res.update({
        "us_per_step": step_us,
        "quantize_q_us": q_us, "decode_us": dec_us, "combine_us": comb_us,
        "kv_bytes": kv_bytes, "algo_bytes_decode": algo,
        "decode_gbps": algo / (dec_us * 1e3),
        "step_kv_gbps": kv_bytes / (step_us * 1e3),
        "decode_mfma_tflops_algorithmic": flops / (dec_us * 1e6),
        "decode_mfma_tflops_executed": flops_exec / (dec_us * 1e6),
        "partial_bytes": B * S * Sq * H * (512 * 2 + 4),
    })
    del pools, po, pl, dw
    torch.cuda.empty_cache()
    return res


def _time_fn_graph(fn, n):
    """Microseconds per call of fn, n calls captured in one HIP graph, replayed in steady
    state (see _time_graph_steady)."""
    import torch
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(n):
            fn()
    return _time_graph_steady(g)[0] * 1e3 / n


def hbm_probes():
    """Measured HBM rates in this run, on the GPU the decode ran on: a streaming read of 1 GiB
    through the library's read probe (and torch's sum over it, for comparison), a device copy
    of 1 GiB (read + write), and the KV-sized
    saturating quantisation through this library (a 2^28-element fp32 tensor, 4 B read + 1 B
    written per element).  These are reference rates, not part of the timed step."""
    import torch
    import fp8_mla_split_amd as mla
    n = 1 << 28
    x = torch.randn(n, device="cuda")
    y = torch.empty_like(x)
    q8 = torch.empty(n, dtype=torch.uint8, device="cuda")
    acc = torch.empty((), device="cuda")

    def timed(fn, reps=10):  # eager launches: each moves 1-5 GiB, launch gaps are noise
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    read_us = timed(lambda: mla.hbm_read_probe(x, sink, 2048))
    sum_us = timed(lambda: torch.sum(x, dim=(0,), out=acc))
    copy_us = timed(lambda: y.copy_(x))
    quant_us = timed(lambda: mla.quantize_fp8_sat(x, 0.01, out=q8))
    res = {"read_gbps": round(4 * n / (read_us * 1e3), 1),
           "torch_sum_read_gbps": round(4 * n / (sum_us * 1e3), 1),
           "copy_gbps": round(8 * n / (copy_us * 1e3), 1),
           "kv_quantize_gbps": round(5 * n / (quant_us * 1e3), 1),
           "kv_quantize_us_per_gi_element": round(quant_us * 4, 1)}
    res["kv_quantize_frac_of_hbm_peak"] = round(res["kv_quantize_gbps"] / HBM_PEAK_GBPS, 4)
    del x, y, q8
    torch.cuda.empty_cache()
    return res


def prep_probes():
    """The cache-preparation entry points, each graph-timed in this run:
    - KV append (mla_kv_append_fp8_sat) at the decode workloads' per-step shapes (one new row
      per request at batch 32; 8 draft rows per request at batch 4) and in bulk (16 requests x
      8192 rows: 4 B read + 1 B written per element, against the HBM roofline);
    - the quantisation with a device-derived scale (mla_quantize_fp8_sat_dynamic) for one
      step's Q at batch 1 and in bulk (2^28 elements, fp32 and bf16 sources).  Its two passes
      read the source twice: algorithmic bytes are one read + one write, the executed traffic
      two reads + one write; both rates are given."""
    import torch
    import fp8_mla_split_amd as mla
    from synthetic import WORKLOADS, q_f32
    res = {}
    rng = np.random.default_rng(0)

    def append_case(batch, t_new, max_pages, page_size=64, reps=200, rope=False):
        pages = batch * max_pages
        pool = torch.zeros((pages, page_size, 576), dtype=torch.uint8, device="cuda")
        table = torch.from_numpy(rng.permutation(pages).astype(np.int32).reshape(
            batch, max_pages)).cuda()
        lens = torch.from_numpy(rng.integers(t_new, max_pages * page_size + 1, size=batch)
                                .astype(np.int32)).cuda()
        new = torch.randn((batch, t_new, 576), device="cuda")
        if rope:  # a standard table: theta_i = 10000^(-2i/64), one row per position
            pos = torch.arange(max_pages * page_size, device="cuda", dtype=torch.float64)
            theta = 10000.0 ** (-torch.arange(32, device="cuda", dtype=torch.float64) / 32.0)
            ang = pos[:, None] * theta[None, :]
            cos_t, sin_t = torch.cos(ang).float(), torch.sin(ang).float()
            fn = lambda: mla.kv_append_rope_fp8_sat(new, pool, table, lens, 0.01, cos_t, sin_t)
        else:
            fn = lambda: mla.kv_append_fp8_sat(new, pool, table, lens, 0.01)
        us = _time_fn_graph(fn, reps)
        return us, batch * t_new * 576
    us, n = append_case(32, 1, 2048)
    res["kv_append_b32_t1_us"] = round(us, 2)
    us, n = append_case(4, 8, 16384)
    res["kv_append_b4_t8_us"] = round(us, 2)
    us, n = append_case(32, 1, 2048, rope=True)
    res["kv_append_rope_b32_t1_us"] = round(us, 2)
    us, n = append_case(4, 8, 16384, rope=True)
    res["kv_append_rope_b4_t8_us"] = round(us, 2)
    us, n = append_case(16, 8192, 129, reps=20)
    res["kv_append_bulk_b16_t8192"] = {"us": round(us, 1), "gbps": round(5 * n / (us * 1e3), 1),
                                       "frac_of_hbm_peak": round(5 * n / (us * 1e3)
                                                                 / HBM_PEAK_GBPS, 4)}
    ws = torch.empty(mla.QUANTIZE_DYNAMIC_WORKSPACE_BYTES // 4, dtype=torch.int32, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    q = torch.from_numpy(q_f32(WORKLOADS["b1_128k"])).cuda()
    q8 = torch.empty(q.shape, dtype=torch.uint8, device="cuda")
    res["dynamic_quantize_q_b1_us"] = round(_time_fn_graph(
        lambda: mla.quantize_fp8_sat_dynamic(q, out=q8, scale=sc, workspace=ws), 200), 2)
    res["host_scale_quantize_q_b1_us"] = round(_time_fn_graph(
        lambda: mla.quantize_fp8_sat(q, 0.01, out=q8), 200), 2)
    n = 1 << 28
    for name, dt, esz in (("f32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
        x = torch.randn(n, device="cuda").to(dt)
        y = torch.empty(n, dtype=torch.uint8, device="cuda")
        us = _time_fn_graph(lambda: mla.quantize_fp8_sat_dynamic(x, out=y, scale=sc,
                                                                 workspace=ws), 5)
        res[f"dynamic_quantize_bulk_{name}"] = {
            "us_per_gi_element": round(us * 4, 1),
            "algorithmic_gbps": round((esz + 1) * n / (us * 1e3), 1),
            "executed_gbps": round((2 * esz + 1) * n / (us * 1e3), 1)}
        del x, y
    torch.cuda.empty_cache()
    return res


def context_parallel_share(key="b1_128k", gpus=8, n=100, sweep=(16, 32, 64, 0)):
    """One GPU's share of a context-parallel decode, at its real shape: every request's KV
    cut into `gpus` contiguous shards (b1_128k: 16,384 of the 131,072 positions); a GPU
    decodes its shard with S_local splits (the shards before the last are told how many
    positions follow them, so that only the last masks causally) and merges them into one
    partial row per query row (mla_splitkv_combine_partial); the GPUs would all-gather those
    rows (reported: B*Sq*H*1028 bytes per GPU, not timed, it needs a second GPU) and run the
    final combine over the `gpus` merged partials (timed).  S_local runs over `sweep` (0 = the
    planner's choice for the shard's length).  The shards rotate over more than 512 MiB of
    KV so that no cache holds them."""
    import torch
    import fp8_mla_split_amd as mla
    from fp8_mla_split_amd.workload import materialize
    from synthetic import WORKLOADS
    w = WORKLOADS[key]
    dw = materialize(w)
    B, Sq, H = w.batch, w.q_tokens, w.heads
    L = int(dw.seq_lens_host.max())
    assert (dw.seq_lens_host == L).all() and dw.kv_pool8.shape[1] == L and L % (32 * gpus) == 0
    Ls = L // gpus
    R = Sq * H
    extra = -(-(512 << 20) // (dw.kv_pool8.numel()))
    copies = [dw.kv_pool8] + [dw.kv_pool8.clone() for _ in range(extra)]
    shards = [c.view(B * gpus, Ls, 576) for c in copies]          # page b * gpus + g
    lens = torch.full((B,), Ls, dtype=torch.int32, device="cuda")
    tables = [(torch.arange(B, dtype=torch.int32, device="cuda") * gpus + g)[:, None]
              .contiguous() for g in range(gpus)]
    after = [torch.full((B,), (gpus - 1 - g) * Ls, dtype=torch.int32, device="cuda")
             if Sq > 1 else None for g in range(gpus)]
    out = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Sq, H), dtype=torch.float32, device="cuda")
    go = torch.empty((B, gpus, R, 512), dtype=torch.float16, device="cuda")
    gl = torch.empty((B, gpus, R), dtype=torch.float32, device="cuda")
    planned = mla.splitkv_plan(B, Sq, H, Ls).num_splits
    rows = []
    for S in sweep:
        S = S or planned
        po = torch.empty((B, S, R, 512), dtype=torch.float16, device="cuda")
        pl = torch.empty((B, S, R), dtype=torch.float32, device="cuda")
        k = [0]

        def decode_share():
            i = k[0]
            k[0] += 1
            c, g = i % len(shards), (i // len(shards)) % gpus
            mla.decode_splitkv(dw.q8, shards[c], tables[g], lens, dw.q_scale, dw.kv_scale,
                               w.softmax_scale, Ls, S, 0, po, pl, ctx_after=after[g])
        for g in range(gpus):  # every GPU's merged partial, as the all-gather would leave them
            mla.decode_splitkv(dw.q8, shards[0], tables[g], lens, dw.q_scale, dw.kv_scale,
                               w.softmax_scale, Ls, S, 0, po, pl, ctx_after=after[g])
            mla.splitkv_combine_partial(po, pl, Sq, H, go[:, g], gl[:, g], gpus * R)
        reps = n if B * Ls <= (1 << 17) else 5
        dec_us = _time_fn_graph(decode_share, reps)
        merge_us = _time_fn_graph(lambda: mla.splitkv_combine_partial(
            po, pl, Sq, H, go[:, 0], gl[:, 0], gpus * R), n)
        comb_us = _time_fn_graph(lambda: mla.splitkv_combine(go, gl, Sq, H, dw.kv_scale,
                                                             out=out, out_lse=lse), n)
        rows.append({"splits_per_shard": S, "planner": S == planned,
                     "share_decode_us": round(dec_us, 2), "local_merge_us": round(merge_us, 2),
                     "final_combine_us": round(comb_us, 2),
                     "share_total_us_without_all_gather": round(dec_us + merge_us + comb_us, 2)})
        del po, pl
    del copies, shards, dw
    torch.cuda.empty_cache()
    return {"workload": w.name, "gpus": gpus, "shard_tokens": Ls,
            "all_gather_bytes_per_gpu": B * R * (512 * 2 + 4), "rows": rows,
            "note": "decode of one GPU's shard, merge of its splits into one partial per "
                    "query row, final combine over all GPUs' merged partials; the all-gather "
                    "of the merged partials between GPUs is not measured (one GPU)"}


def step_percentiles(key, n_steps=60):
    """p10 / p50 / p90 of single decode steps (quantize + decode + combine), each a one-step
    HIP graph on its own KV copy (so no step finds its KV cached), timed with events."""
    import torch
    import fp8_mla_split_amd as mla
    from fp8_mla_split_amd.workload import materialize
    from synthetic import WORKLOADS, q_f32

    w = WORKLOADS[key]
    dw = materialize(w)
    kv_bytes = dw.kv_tokens * 576
    copies = max(2, -(-(512 << 20) // max(kv_bytes, 1)) + 1) if kv_bytes < (512 << 20) else 2
    pools = [dw.kv_pool8] + [dw.kv_pool8.clone() for _ in range(copies - 1)]
    q32 = torch.from_numpy(q_f32(w)).cuda()
    q8 = torch.empty_like(q32, dtype=torch.uint8)
    plan = mla.splitkv_plan(w.batch, w.q_tokens, w.heads, dw.max_seq_len,
                            total_kv_tokens=dw.kv_tokens)
    S = plan.num_splits
    po = torch.empty((w.batch, S, w.q_tokens * w.heads, 512), dtype=torch.float16, device="cuda")
    pl = torch.empty((w.batch, S, w.q_tokens * w.heads), dtype=torch.float32, device="cuda")
    out = torch.empty((w.batch, w.q_tokens, w.heads, 512), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    graphs = []
    for i in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            mla.quantize_fp8_sat(q32, dw.q_scale, out=q8)
            mla.decode_splitkv(q8, pools[i], dw.page_table, dw.seq_lens, dw.q_scale, dw.kv_scale,
                               w.softmax_scale, dw.max_seq_len, S, 0, po, pl)
            mla.splitkv_combine(po, pl, w.q_tokens, w.heads, dw.kv_scale, out=out)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    ts = []
    with torch.cuda.stream(stream):
        for k in range(n_steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graphs[k % copies].replay()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
    p10, p50, p90 = np.percentile(ts, [10, 50, 90])
    del graphs, pools, dw
    torch.cuda.empty_cache()
    return {"workload": w.name, "steps": n_steps, "p10_us": round(float(p10), 2),
            "p50_us": round(float(p50), 2), "p90_us": round(float(p90), 2),
            "note": "one-step graph replays, each launched and timed on its own (includes "
                    "the graph launch latency that back-to-back steps overlap)"}


def split_sweep(key, splits=(8, 16, 32, 64, 128, 256, 512), n=40):
    """Decode + combine time at fixed split counts beside the planner's choice (graph-timed,
    KV copies rotated as in the main measurement)."""
    import torch
    import fp8_mla_split_amd as mla
    from fp8_mla_split_amd.workload import materialize
    from synthetic import WORKLOADS

    w = WORKLOADS[key]
    dw = materialize(w)
    kv_bytes = dw.kv_tokens * 576
    copies = max(1, -(-(512 << 20) // max(kv_bytes, 1)) + 1) if kv_bytes < (512 << 20) else 1
    pools = [dw.kv_pool8] + [dw.kv_pool8.clone() for _ in range(copies - 1)]
    plan = mla.splitkv_plan(w.batch, w.q_tokens, w.heads, dw.max_seq_len,
                            total_kv_tokens=dw.kv_tokens)
    rows = []
    for S in sorted(set(splits) | {plan.num_splits}):
        po = torch.empty((w.batch, S, w.q_tokens * w.heads, 512), dtype=torch.float16,
                         device="cuda")
        pl = torch.empty((w.batch, S, w.q_tokens * w.heads), dtype=torch.float32, device="cuda")
        out = torch.empty((w.batch, w.q_tokens, w.heads, 512), dtype=torch.bfloat16, device="cuda")
        it = [0]

        def one():
            mla.decode_splitkv(dw.q8, pools[it[0] % copies], dw.page_table, dw.seq_lens,
                               dw.q_scale, dw.kv_scale, w.softmax_scale, dw.max_seq_len, S, 0,
                               po, pl)
            mla.splitkv_combine(po, pl, w.q_tokens, w.heads, dw.kv_scale, out=out)
            it[0] += 1
        us = _time_fn_graph(one, n)
        rows.append({"splits": S, "decode_plus_combine_us": round(us, 2),
                     "planner": S == plan.num_splits})
        del po, pl, out
    del pools, dw
    torch.cuda.empty_cache()
    return {"workload": w.name, "rows": rows}


def cpu_baseline(key, budget_s):
    """The oracle as it stands, one decode step at a time on the host cores, until about
    budget_s seconds of work are done (the sample is a count of whole steps of request 0)."""
    from oracle import attention_fp64, per_tensor_scale, quantize_e4m3_sat
    from synthetic import WORKLOADS, kv_request_f32, page_layout, q_f32, seq_lens_for

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
        if el >= budget_s or n >= 200:
            break
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        cores = max(int(i.get("num_threads", 1)) for i in info)
        blas = ", ".join(f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                         for i in info)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    us = el / n * 1e6 * w.batch  # the oracle handles requests one after another
    return {"value": round(us, 1), "unit": "us/step", "cores": cores, "kind": "oracle",
            "blas": blas,
            "sample": f"{n} full decode steps of request 0 of {w.name} (Q quantize + fp64 "
                      f"attention over all {int(lens[0])} positions and {w.heads} heads), "
                      f"{el:.1f} s of host time"}


def decode_source_hash():
    """sha256[:16] of decode.hip without its // comments and blank space, so that the record
    of counters survives comment edits but not code changes (the source has no "//" inside
    string literals)."""
    import re
    with open(os.path.join(ROOT, "fp8_mla_split_amd", "csrc", "decode.hip")) as f:
        code = re.sub(r"//[^\n]*", "", f.read())
    code = "\n".join(" ".join(line.split()) for line in code.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed profiler counters, if they were taken
    on the decode kernel as it is now (same source hash) and on this workload; else None."""
    path = os.path.join(ROOT, "profiles", "decode_kernel_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("decode_source_sha256_16") != decode_source_hash():
        return None
    return rec.get("bytes_per_launch", {}).get(workload)


def main():
    a = _parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              f"(how the path would shard over GPUs is described, not built)", file=sys.stderr)
        sys.exit(2)
    if a.copy_probe_mib:
        copy_probe(a.copy_probe_mib, a.steps)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    sys.path.insert(0, ROOT)
    if a.prep_only:
        print(json.dumps({"cache_prep": prep_probes()}), flush=True)
        return
    if a.cp_workload:
        print(json.dumps({"context_parallel_share": context_parallel_share(
            a.cp_workload, sweep=(0,) if a.cp_workload != "b1_128k" else (16, 32, 64, 0))}),
            flush=True)
        return
    t_wall = time.time()
    q_lens = [int(x) for x in a.q_lens.split(",")] if a.q_lens else None
    main_res = run_workload(a.workload, a.steps, a.warmup, a.splits, a.rows_per_group, a.eager,
                            q_lens=q_lens, longest_first=a.order == "longest")
    print(f"[bench] {a.workload}: {main_res['us_per_step']:.2f} us/step (decode "
          f"{main_res['decode_us']:.2f} us, {main_res['decode_gbps']:.0f} GB/s; combine "
          f"{main_res['combine_us']:.2f} us; Q quantize {main_res['quantize_q_us']:.2f} us)",
          file=sys.stderr, flush=True)
    also = None
    if a.also:
        also = run_workload(a.also, max(20, a.steps // 4), max(5, a.warmup // 4), 0, 0, a.eager)
        print(f"[bench] {a.also}: {also['us_per_step']:.2f} us/step (decode "
              f"{also['decode_us']:.2f} us, {also['decode_gbps']:.0f} GB/s)",
              file=sys.stderr, flush=True)
    extras = None
    if not a.no_extras:
        extras = {"hbm_probes": hbm_probes(),
                  "step_percentiles": step_percentiles(a.workload),
                  "split_sweep": split_sweep(a.workload),
                  "cache_prep": prep_probes(),
                  "context_parallel_share": context_parallel_share()}
        others = {}
        for key, kw in (("paged_b32", {"longest_first": True}), ("verify_b4_1m", {})):
            r = run_workload(key, 20, 3, 0, 0, a.eager, **kw)
            others[key] = {k: (round(r[k], 3) if isinstance(r[k], float) else r[k]) for k in (
                "us_per_step", "decode_us", "combine_us", "num_splits", "kv_tokens",
                "decode_gbps", "decode_mfma_tflops_algorithmic", "decode_mfma_tflops_executed")}
            others[key]["decode_frac_of_hbm_peak"] = round(r["decode_gbps"] / HBM_PEAK_GBPS, 4)
            if kw:
                others[key]["order"] = "longest first"
            print(f"[bench] {key}: {r['us_per_step']:.1f} us/step (decode {r['decode_us']:.1f} "
                  f"us)", file=sys.stderr, flush=True)
        extras["other_workloads"] = others
        dyn = run_workload(a.workload, a.steps, a.warmup, a.splits, a.rows_per_group, a.eager,
                           dev_scales=True)
        extras["device_scale_step"] = {k: round(dyn[k], 3) for k in (
            "us_per_step", "quantize_q_us", "decode_us", "combine_us")}
        extras["device_scale_step"]["note"] = (
            "the same step with Q's scale derived on the GPU and both scales read by the "
            "decode and combine from device memory")
        print(f"[bench] device-scale step: {dyn['us_per_step']:.2f} us (Q amax+quantize "
              f"{dyn['quantize_q_us']:.2f} us); cache prep: "
              + json.dumps(extras["cache_prep"]), file=sys.stderr, flush=True)
        pr = extras["hbm_probes"]
        print(f"[bench] measured HBM: read {pr['read_gbps']:.0f} GB/s, copy {pr['copy_gbps']:.0f} "
              f"GB/s, KV quantize {pr['kv_quantize_gbps']:.0f} GB/s; step p10/p50/p90 "
              f"{extras['step_percentiles']['p10_us']}/{extras['step_percentiles']['p50_us']}/"
              f"{extras['step_percentiles']['p90_us']} us", file=sys.stderr, flush=True)
        print("[bench] split sweep: " + ", ".join(
            f"S={r['splits']}{'*' if r['planner'] else ''} {r['decode_plus_combine_us']:.1f} us"
            for r in extras["split_sweep"]["rows"]), file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(a.workload, a.cpu_seconds)
    achieved = main_res["decode_gbps"]
    traffic = measured_traffic(main_res["workload"])
    line = {
        "metric": METRIC,
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
                                            "num_splits", "rows_per_group", "kv_copies",
                                            "timing")} | {
            k: main_res[k] for k in ("q_lens", "order") if k in main_res},
        "kv_read_gbps_step": round(main_res["step_kv_gbps"], 1),
        "kv_read_pct_of_peak_step": round(100 * main_res["step_kv_gbps"] / HBM_PEAK_GBPS, 2),
        "breakdown_us": {k: round(main_res[k], 3) for k in ("quantize_q_us", "decode_us",
                                                            "combine_us")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "decode_kernel (mla_decode_splitkv)",
                     "algorithmic_bytes_per_launch": main_res["algo_bytes_decode"],
                     "mfma_tflops_algorithmic": round(main_res["decode_mfma_tflops_algorithmic"], 1),
                     "mfma_tflops_executed": round(main_res["decode_mfma_tflops_executed"], 1),
                     "mfma_peak_tflops_fp8": FP8_PEAK_TFLOPS},
        "cpu_baseline": cpu,
        "decode_frac_of_measured_read_peak": None if extras is None else round(
            achieved / extras["hbm_probes"]["read_gbps"], 4),
        "extras": extras,
        "also": None if also is None else {
            "workload": also["workload"], "us_per_step": round(also["us_per_step"], 3),
            "decode_us": round(also["decode_us"], 3),
            "combine_us": round(also["combine_us"], 3),
            "decode_gbps": round(also["decode_gbps"], 1),
            "decode_frac_of_hbm_peak": round(also["decode_gbps"] / HBM_PEAK_GBPS, 4),
            "step_kv_gbps": round(also["step_kv_gbps"], 1),
            "decode_mfma_tflops_algorithmic": round(also["decode_mfma_tflops_algorithmic"], 1),
            "decode_mfma_tflops_executed": round(also["decode_mfma_tflops_executed"], 1),
            "decode_mfma_frac_of_fp8_peak_executed": round(
                also["decode_mfma_tflops_executed"] / FP8_PEAK_TFLOPS, 4),
            "num_splits": also["num_splits"], "rows_per_group": also["rows_per_group"]},
        "detail": main_res,
        "wall_s": round(time.time() - t_wall, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
