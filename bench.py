#!/usr/bin/env python3
"""Benchmark of NVFP4 paged attention on one MI355X.

Default workload: batch decode (64 requests, kv_len ~ U[512, 8192], 32 qo / 8 kv heads,
head dim 128, page size 16, 40k-page pool in a seeded random permutation, split-KV
with 256-token chunks).  One step = append the step's new K/V token of every request
(NVFP4 quantise into its slot) + the decode over the paged cache (split chunks merged
by LSE).  The plan is built once (the lengths do not change between steps) and its
host time is reported separately.  Inputs are resident in HBM before timing starts;
three independent pool sets are rotated so that the 256 MB Infinity Cache cannot
serve a step from the previous one.

Prints one JSON line.  ``value`` is the decode's KV GB/s (packed e2m1 bytes plus e4m3
scale bytes of every visible K and V row, divided by the step time).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="batch_decode")
    p.add_argument("--pool-sets", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads' lines")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    return p.parse_args()


def time_events(torch, fn, iters):
    """Average duration (ms) of fn() over iters launches, HIP events on the current stream."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def decode_bytes(w):
    q = w.batch * w.num_qo_heads * w.head_dim_qk * 2
    o = w.batch * w.num_qo_heads * (w.head_dim_vo * 4 + 4)
    return w.kv_bytes(), q + o


def cpu_baseline(torch, case, budget_s):
    """The oracle on a bounded sample of the same decode workload (one BLAS thread)."""
    from threadpoolctl import threadpool_limits
    from oracle import nvfp4_ref as ref
    from attention_bit_paged_amd import synth
    w = case.w
    kd, ks = case.k_pool.data.cpu().numpy(), case.k_pool.sf.cpu().numpy()
    vd, vs = case.v_pool.data.cpu().numpy(), case.v_pool.sf.cpu().numpy()
    q = case.q.float().cpu().double().numpy()
    ind = synth.indptr(w.qo_lens)
    done, nbytes = [], 0
    per_tok = w.num_kv_heads * (w.head_dim_qk // 2 + w.head_dim_qk // 16 + w.head_dim_vo // 2
                                + w.head_dim_vo // 16)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for b in range(w.batch):
            ref.paged_attention(q, kd, ks, vd, vs, case.page_table_np, w.kv_lens, ind, w.page_size,
                                w.sm_scale, False, "HND", rows=[b])
            done.append(b)
            nbytes += w.kv_lens[b] * per_tok
            if time.perf_counter() - t0 > budget_s and len(done) >= 2:
                break
        dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(done)} of {w.batch} requests ({sum(w.kv_lens[b] for b in done)} "
                      f"tokens x {w.num_kv_heads} kv heads), numpy float64, {dt:.1f} s"}


def extra_decode(torch, nv, paged, synth, name, iters=20):
    w = synth.workload(name)
    case = paged.build_case(w, keep_sources=False)
    plan = paged.make_plan(case)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.empty((w.batch, w.num_qo_heads, w.head_dim_vo), device="cuda")
    lse = torch.empty((w.batch, w.num_qo_heads), device="cuda")
    fn = lambda: nv.batch_decode(plan, case.q, case.page_table, case.k_pool, case.v_pool,
                                 w.sm_scale, ws, out=o, lse=lse)
    for _ in range(3):
        fn()
    ms = time_events(torch, fn, iters)
    kv, _ = decode_bytes(w)
    info = plan.info()
    del case, ws
    torch.cuda.empty_cache()
    return {"workload": name, "kv_GBs": round(kv / ms / 1e6, 1),
            "frac_hbm": round(kv / ms / 1e6 / HBM_PEAK_GBS, 4), "ms": round(ms, 4),
            "kv_bytes": kv, "chunk": info["kv_chunk_tokens"], "work_items": info["num_work_items"]}


def extra_prefill(torch, nv, paged, synth, name, iters=10):
    w = synth.workload(name)
    case = paged.build_case(w, keep_sources=False)
    plan = paged.make_plan(case)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim_vo), device="cuda")
    lse = torch.empty((w.total_q, w.num_qo_heads), device="cuda")
    fn = lambda: nv.batch_prefill(plan, case.q, case.page_table, case.k_pool, case.v_pool,
                                  w.sm_scale, ws, out=o, lse=lse)
    for _ in range(3):
        fn()
    ms = time_events(torch, fn, iters)
    fl = w.flops()
    info = plan.info()
    del case, ws
    torch.cuda.empty_cache()
    return {"workload": name, "TFLOPs": round(fl / ms / 1e9, 2),
            "frac_mfma_f16": round(fl / ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4), "ms": round(ms, 4),
            "flops": fl, "work_items": info["num_work_items"], "chunk": info["kv_chunk_tokens"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by request or kv head with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import attention_bit_paged_amd as nv
    from attention_bit_paged_amd import paged, synth

    w = synth.workload(args.workload)
    if not w.decode:
        raise SystemExit("the timed step is the decode workload; prefill runs as an extra line")
    sets = [paged.build_case(w, keep_sources=(i == 0)) for i in range(args.pool_sets)]
    case0 = sets[0]
    t0 = time.perf_counter()
    plan = paged.make_plan(case0)
    plan_us = (time.perf_counter() - t0) * 1e6
    ws = plan.new_workspace()
    plan.upload(ws)
    info = plan.info()

    # the step's new token of every request: its K/V rows and the slot of token L_b - 1
    g = torch.Generator(device="cuda")
    g.manual_seed(w.value_seed + 500)
    new_k = torch.randn((w.batch, w.num_kv_heads, w.head_dim_qk), generator=g, device="cuda").bfloat16()
    new_v = torch.randn((w.batch, w.num_kv_heads, w.head_dim_vo), generator=g, device="cuda").bfloat16()
    last = []
    pos = 0
    for L in w.kv_lens:
        pos += L
        last.append(pos - 1)
    new_slots = case0.slots[torch.tensor(last, device="cuda")]
    o = torch.empty((w.batch, w.num_qo_heads, w.head_dim_vo), device="cuda")
    lse = torch.empty((w.batch, w.num_qo_heads), device="cuda")

    def step(i):
        c = sets[i % len(sets)]
        nv.quantize_kv(new_k, new_v, new_slots, c.k_pool, c.v_pool)
        nv.batch_decode(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o, lse=lse)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps

    # per-kernel HIP-event timing on the launch stream (same rotation as the steps)
    ctr = [0]

    def dec():
        c = sets[ctr[0] % len(sets)]
        ctr[0] += 1
        nv.batch_decode(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o, lse=lse)

    def quant():
        c = sets[ctr[0] % len(sets)]
        ctr[0] += 1
        nv.quantize_kv(new_k, new_v, new_slots, c.k_pool, c.v_pool)

    dec_ms = time_events(torch, dec, max(args.steps, 20))
    quant_ms = time_events(torch, quant, max(args.steps, 20))

    kv, qo = decode_bytes(w)
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = (kv + qo) / (dec_ms * 1e-3) / 1e9
    out = {
        "metric": "NVFP4 paged decode KV GB/s (% HBM peak); prefill TFLOP/s (% MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 KV (e2m1 + e4m3), fp16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, NVFP4-quantised in-kernel)",
        "config": {"workload": w.name, "batch": w.batch, "kv_len": "U[512,8192] seeded",
                   "num_qo_heads": w.num_qo_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim_qk, "page_size": w.page_size, "pool_pages": w.pool_pages,
                   "kv_chunk_tokens": info["kv_chunk_tokens"], "work_items": info["num_work_items"],
                   "total_kv_tokens": w.total_kv, "pool_sets_rotated": len(sets)},
        "frac_hbm": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "decode (decode_kernel + merge_partials_kernel)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": kv + qo, "avg_launch_ms": round(dec_ms, 5)},
        "quantize_append_ms": round(quant_ms, 5),
        "plan_host_us": round(plan_us, 1),
    }
    if not args.no_extra:
        extras = []
        for name in ("long_decode", "asym_decode"):
            extras.append(extra_decode(torch, nv, paged, synth, name))
        for name in ("prefill_extend", "asym_prefill"):
            extras.append(extra_prefill(torch, nv, paged, synth, name))
        out["other_workloads"] = extras
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(torch, case0, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
