#!/usr/bin/env python3
"""Benchmark of NVFP4 paged attention on one MI355X.

Default workload: batch decode (64 requests, kv_len ~ U[512, 8192], 32 qo / 8 kv heads,
head dim 128, page size 16, 40k-page pool in a seeded random permutation, split-KV
with 256-token chunks).  One step = append the step's new K/V token of every request
(NVFP4 quantise into the slot of its last key) + the attention pass over the paged
cache, both in one launch (nvfp4_batch_decode_append), + the LSE merge of the split
rows.  The same step with the append as its own launch is timed for the breakdown.
The plan is built once (the lengths do not change between steps) and its host time
is reported separately.  Inputs are resident in HBM before
timing starts; three independent pool sets are rotated so that the 256 MB Infinity
Cache cannot serve a step from the previous one.

Prints one JSON line.  ``value`` is the decode's KV GB/s: packed e2m1 bytes plus e4m3
scale bytes of every visible K and V row, divided by the step time.  ``roofline`` is
the attention kernel's own figure: its algorithmic bytes (KV + Q + O + LSE + the new
token's rows) over its average duration, timed inside the timed steps with HIP events
that the kernel's dispatch itself timestamps (nvfp4_set_timing_events), so that no
event packet is added to the queue.

Also in the line (default run): ``stream_ceiling``, the same plan's KV bytes streamed
through the same rings and copies with no attention arithmetic (nvfp4_kv_checksum),
timed the same way: what the access pattern itself sustains; ``single_decode_latency``,
percentiles of one 128-key single-request decode (kernel and call-to-completion);
``cpu_baseline``, the oracle on a bounded sample of the workload on one host thread and
on the host's threads; ``other_workloads``, the long-context and 512/256 decodes and the
two prefills, each with its own CPU baseline (and streaming ceiling for the decodes).

With --workload naming a prefill workload, the timed step is that prefill's attention
pass and merge instead (TFLOP/s; used to profile the prefill kernel).

Other modes (profiling support):
  --pmc-run                a short program for rocprofv3 counter passes: a 1 GiB copy
                           (counter calibration) and a few steps of the workload (with
                           --variant: a few plain decode launches of that layout variant);
  --summarize-trace DIR    summarise a rocprofv3 --kernel-trace --stats output dir;
  --summarize-pmc DIR ...  summarise FETCH_SIZE / WRITE_SIZE counter dirs into the
                           traffic record read back by the benchmark;
  --summarize-counters DIR ...  summarise SQ counter passes of one kernel (--kernel
                           names it): MFMA busy share, instruction mix per wave, waits.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
# sources whose change invalidates recorded counters of the decode kernel
DECODE_SOURCES = ("decode.hip", "kv_ring.h", "attn_step.h", "fp4_common.h", "fp4_quant.h",
                  "internal.h")
CALIB_BYTES = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # defaults: about 50 ms of timed decode steps after the clocks and queues have
    # reached their steady state (10 warmup steps measured 3-4 % below it)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="batch_decode")
    p.add_argument("--pool-sets", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads' lines")
    # per leg (one thread, then the host threads) and workload: about 2 x 5 x 3 s of
    # oracle work in the default run
    p.add_argument("--cpu-seconds", type=float, default=3.0)
    p.add_argument("--pmc-run", action="store_true")
    p.add_argument("--variant", default="", help="layout variant of --pmc-run (a VARIANTS label)")
    p.add_argument("--summarize-trace", metavar="DIR")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR")
    p.add_argument("--kernel", default="prefill_coop_kernel", help="kernel of --summarize-counters")
    p.add_argument("--command", default="", help="command line recorded in a summary")
    p.add_argument("--out", default="", help="summary file to write")
    return p.parse_args()


def sources_digest():
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "attention_bit_paged_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_record_path(workload):
    return os.path.join(PROFILES, f"decode_ring_kernel.{workload}.traffic.txt")


def recorded_traffic(workload):
    """HBM bytes per launch of the decode kernel from the committed counter record, or
    None when there is none or the kernel sources changed since it was taken."""
    path = traffic_record_path(workload)
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("{"):
                rec = json.loads(line)
    if not rec or rec.get("source_digest") != sources_digest():
        return None
    return rec["bytes_per_launch"]


class HipEvents:
    """Timing events created directly through HIP, without the system-scope fence a
    default event performs when it is recorded (that fence adds several microseconds
    to every bracketed launch)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.pool = []

    def new(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e),
                                            self.ct.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.pool.append(e)
        return e

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    @staticmethod
    def time_launches(nv, start, stop):
        """Attention launches from now on carry (start, stop), timestamped by the dispatch
        itself (nvfp4_set_timing_events); None, None stops."""
        nv.check(nv.lib.nvfp4_set_timing_events(start, stop))

    def ms(self, a, b):
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def __del__(self):
        for e in self.pool:
            self.hip.hipEventDestroy(e)


def decode_bytes(w, append=False):
    """(KV bytes, other bytes) of one decode launch: Q read, O and LSE written, and with
    ``append`` the new token's bf16 rows read and their NVFP4 bytes written."""
    q = w.batch * w.num_qo_heads * w.head_dim_qk * 2
    o = w.batch * w.num_qo_heads * (w.head_dim_vo * 4 + 4)
    new = 0
    if append:
        dk, dv = w.head_dim_qk, w.head_dim_vo
        new = w.batch * w.num_kv_heads * (2 * (dk + dv) + dk // 2 + dk // 16 + dv // 2 + dv // 16)
    return w.kv_bytes(), q + o + new


def _pair_work(w, b):
    """Algorithmic work of one (request, kv head) pair: KV bytes (decode) or flops."""
    if w.decode:
        return w.kv_lens[b] * (w.head_dim_qk // 2 + w.head_dim_qk // 16 + w.head_dim_vo // 2
                               + w.head_dim_vo // 16)
    q, l = w.qo_lens[b], w.kv_lens[b]
    pairs = q * (l - q) + q * (q + 1) // 2 if w.causal else q * l
    return 2 * (w.head_dim_qk + w.head_dim_vo) * w.group * pairs


def cpu_threads():
    """Host threads for the oracle's parallel leg: the host's cores, at most 16 (the
    share of one GPU's host on a shared machine)."""
    return max(1, min(os.cpu_count() or 1, 16))


def cpu_baseline(case, budget_s, threads):
    """The oracle (numpy float64, as it stands) on a bounded, seeded sample of the same
    workload's (request, kv head) pairs, run from the pools' bytes.  Timed twice: on one
    thread, and on ``threads`` host threads, each computing whole pairs (BLAS held to
    one thread per pair, so the threads are the cores used).  Each leg stops taking new
    pairs after ``budget_s``; its rate over the pairs done stands for the workload."""
    import itertools
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait
    from threadpoolctl import threadpool_limits
    from oracle import nvfp4_ref as ref
    from attention_bit_paged_amd import synth
    w = case.w
    kd, ks = case.k_pool.data.cpu().numpy(), case.k_pool.sf.cpu().numpy()
    vd, vs = case.v_pool.data.cpu().numpy(), case.v_pool.sf.cpu().numpy()
    q = case.q.float().cpu().double().numpy()
    ind = synth.indptr(w.qo_lens)
    g = w.group
    order = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    order = [order[i] for i in np.random.default_rng(7).permutation(len(order))]
    total = sum(_pair_work(w, b) for b, _ in order)

    def one(pair):
        b, h = pair
        ref.paged_attention(q[:, g * h:g * (h + 1)], kd[:, h:h + 1], ks[:, h:h + 1],
                            vd[:, h:h + 1], vs[:, h:h + 1], case.page_table_np, w.kv_lens, ind,
                            w.page_size, w.sm_scale, w.causal, "HND", rows=[b])
        return _pair_work(w, b)

    def leg(n):
        """Pairs done, their work and the elapsed time on n threads; no new pair starts
        after budget_s."""
        done, work = 0, 0
        with threadpool_limits(1), ThreadPoolExecutor(n) as ex:
            t0 = time.perf_counter()
            pending = iter(order)
            running = {ex.submit(one, p) for p in itertools.islice(pending, n)}
            while running:
                finished, running = wait(running, return_when=FIRST_COMPLETED)
                for f in finished:
                    work += f.result()
                    done += 1
                    if time.perf_counter() - t0 <= budget_s:
                        p = next(pending, None)
                        if p is not None:
                            running.add(ex.submit(one, p))
            dt = time.perf_counter() - t0
        return done, work, dt

    unit, scale = ("GB/s", 1e9) if w.decode else ("GFLOP/s", 1e9)
    d1, w1, t1 = leg(1)
    dn, wn, tn = leg(threads)
    return {"workload": w.name, "unit": unit,
            "value_1_thread": round(w1 / t1 / scale, 4),
            "value_threads": round(wn / tn / scale, 4), "threads": threads,
            "sample_1_thread": f"{d1} of {len(order)} (request, kv head) pairs, "
                               f"{100 * w1 / total:.2f} % of the work, {t1:.1f} s",
            "sample_threads": f"{dn} of {len(order)} pairs, {100 * wn / total:.2f} % of the "
                              f"work, {tn:.1f} s",
            "full_workload_s_extrapolated": round(total / (wn / tn), 1)}


def timed_passes(torch, nv, run, merge, iters):
    """Per-launch durations (ms) of the attention kernel (events carried by its dispatch)
    and of the merge (events recorded around it).  ``run`` and ``merge`` may be lists
    (one call per pool set), taken in turn."""
    runs = run if isinstance(run, (list, tuple)) else [run]
    merges = merge if isinstance(merge, (list, tuple)) else [merge]
    s = torch.cuda.current_stream()
    he = HipEvents()
    ev = [[he.new() for _ in range(4)] for _ in range(iters)]
    for i, e in enumerate(ev):
        he.time_launches(nv, e[0], e[1])
        runs[i % len(runs)]()
        he.time_launches(nv, None, None)
        he.record(e[2], s)
        merges[i % len(merges)]()
        he.record(e[3], s)
    torch.cuda.synchronize()
    return (float(np.mean([he.ms(e[0], e[1]) for e in ev])),
            float(np.mean([he.ms(e[2], e[3]) for e in ev])))


def extra_decode(torch, nv, paged, synth, name, iters=100, warm=20, cpu_budget=0.0,
                 pool_sets=3):
    """One decode workload's line, over ``pool_sets`` rotated pool sets like the main line
    (a workload smaller than the 256 MB Infinity Cache would otherwise be read from it)."""
    w = synth.workload(name)
    cases = [paged.build_case(w, keep_sources=False) for _ in range(pool_sets)]
    case = cases[0]
    plan = paged.make_plan(case)
    plan.set_deferred_merge(True)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.empty((w.batch, w.num_qo_heads, w.head_dim_vo), device="cuda")
    lse = torch.empty((w.batch, w.num_qo_heads), device="cuda")
    run = [nv.batch_decode(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o,
                           lse=lse, prepare=True) for c in cases]
    merge = nv.merge_partials(plan, ws, o, lse, prepare=True)
    for i in range(warm):
        run[i % pool_sets]()
        merge()
    run_ms, merge_ms = timed_passes(torch, nv, run, merge, iters)
    del run, merge
    kv, qo = decode_bytes(w)
    info = plan.info()
    out = {"workload": name, "kv_GBs": round(kv / (run_ms + merge_ms) / 1e6, 1),
           "kernel_GBs": round((kv + qo) / run_ms / 1e6, 1),
           "kernel_frac_hbm": round((kv + qo) / run_ms / 1e6 / HBM_PEAK_GBS, 4),
           "attn_ms": round(run_ms, 4), "merge_ms": round(merge_ms, 4), "kv_bytes": kv,
           "chunk": info["kv_chunk_tokens"], "work_items": info["num_work_items"],
           "pool_sets_rotated": pool_sets}
    if w.page_size >= 16:
        out["stream_ceiling"] = stream_ceiling(torch, nv, plan, cases, ws, iters, kv, run_ms)
    if cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(case, cpu_budget, cpu_threads())
    del case, cases, ws
    torch.cuda.empty_cache()
    return out


def extra_prefill(torch, nv, paged, synth, name, iters=40, warm=40, cpu_budget=0.0,
                  pool_sets=3):
    """One prefill workload's line.  The first prefill line of a run follows the decode
    lines; with ten warm-up passes it measured about 8 % below the same kernel timed
    later in the run, so the warm-up is forty passes."""
    w = synth.workload(name)
    cases = [paged.build_case(w, keep_sources=False) for _ in range(pool_sets)]
    case = cases[0]
    plan = paged.make_plan(case)
    plan.set_deferred_merge(True)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim_vo), device="cuda")
    lse = torch.empty((w.total_q, w.num_qo_heads), device="cuda")
    run = [nv.batch_prefill(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o,
                            lse=lse, prepare=True) for c in cases]
    merge = nv.merge_partials(plan, ws, o, lse, prepare=True)
    for i in range(warm):
        run[i % pool_sets]()
        merge()
    run_ms, merge_ms = timed_passes(torch, nv, run, merge, iters)
    del run, merge
    fl = w.flops()
    info = plan.info()
    out = {"workload": name, "TFLOPs": round(fl / (run_ms + merge_ms) / 1e9, 2),
           "kernel_TFLOPs": round(fl / run_ms / 1e9, 2),
           "kernel_frac_mfma_f16": round(fl / run_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
           "attn_ms": round(run_ms, 4), "merge_ms": round(merge_ms, 4), "flops": fl,
           "work_items": info["num_work_items"], "chunk": info["kv_chunk_tokens"],
           "pool_sets_rotated": pool_sets}
    if cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(case, cpu_budget, cpu_threads())
    del case, cases, ws
    torch.cuda.empty_cache()
    return out


# Layout variants of the batch decode and the prefill extend, each against the HND,
# page size 16, dense-stride line measured the same way: (label, layout, page size,
# K parent padding, V parent padding).  The padding makes K's and V's strides differ
# from a dense pool's and from each other's.
VARIANTS = (("HND_page16", "HND", 16, None, None),
            ("NHD_page16", "NHD", 16, None, None),
            ("HND_page16_unequal_strides", "HND", 16, (1, 1, 3, 16), (2, 0, 1, 32)),
            ("HND_page1", "HND", 1, None, None))


def variant_workload(synth, name, label):
    """The workload under layout variant ``label`` and its (layout, K, V padding)."""
    base = synth.workload(name)
    for lab, layout, ps, kp, vp in VARIANTS:
        if lab == label:
            w = synth.workload(name, page_size=ps,
                               pool_pages=base.pool_pages * base.page_size // ps)
            return w, layout, kp, vp
    raise SystemExit(f"unknown variant {label!r}; one of {[v[0] for v in VARIANTS]}")


def variant_case(paged, synth, name, label):
    w, layout, kp, vp = variant_workload(synth, name, label)
    case = paged.build_case(w, keep_sources=False, layout=layout, k_pad=kp, v_pad=vp)
    return w, case, paged.make_plan(case)


def variant_lines(torch, nv, paged, synth, name, iters=60, warm=12, pool_sets=3):
    """Kernel throughput of one workload under each layout variant (same values, same
    request lengths; the page size changes the pool's page count, not its bytes), over
    ``pool_sets`` rotated pool sets like the main line."""
    lines, ref_rate = [], None
    for label, *_ in VARIANTS:
        w, layout, kp, vp = variant_workload(synth, name, label)
        cases = [paged.build_case(w, keep_sources=False, layout=layout, k_pad=kp, v_pad=vp)
                 for _ in range(pool_sets)]
        case = cases[0]
        plan = paged.make_plan(case)
        plan.set_deferred_merge(True)
        ws = plan.new_workspace()
        plan.upload(ws)
        o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim_vo), device="cuda")
        lse = torch.empty((w.total_q, w.num_qo_heads), device="cuda")
        fn = nv.batch_decode if w.decode else nv.batch_prefill
        run = [fn(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o, lse=lse,
                  prepare=True) for c in cases]
        merge = nv.merge_partials(plan, ws, o, lse, prepare=True)
        for i in range(warm):
            run[i % len(run)]()
            merge()
        run_ms, _ = timed_passes(torch, nv, run, merge, iters)
        if w.decode:
            kv, qo = decode_bytes(w)
            rate = (kv + qo) / run_ms / 1e6
            line = {"variant": label, "kernel_GBs": round(rate, 1),
                    "kernel_frac_hbm": round(rate / HBM_PEAK_GBS, 4)}
        else:
            rate = w.flops() / run_ms / 1e9
            line = {"variant": label, "kernel_TFLOPs": round(rate, 2),
                    "kernel_frac_mfma_f16": round(rate / MFMA_F16_PEAK_TFLOPS, 4)}
        ref_rate = rate if ref_rate is None else ref_rate
        line.update(attn_ms=round(run_ms, 4), vs_HND_page16=round(rate / ref_rate, 4),
                    k_strides=[case.k_pool.struct().stride_page, case.k_pool.struct().stride_head,
                               case.k_pool.struct().stride_token],
                    v_strides=[case.v_pool.struct().stride_page, case.v_pool.struct().stride_head,
                               case.v_pool.struct().stride_token])
        lines.append(line)
        del run, merge, case, cases, ws
        torch.cuda.empty_cache()
    return {"workload": name, "lines": lines}


def kv_type_lines(torch, nv, paged, synth, iters=60, warm=12, pool_sets=3):
    """The FP8 e4m3 cache beside NVFP4 (batch decode, 512/256 decode, prefill extend), and
    the prefill extend over ragged (non-paged) rows of either type; kernel figures as in
    the main lines (decode: the type's own KV bytes + Q + O + LSE; prefill: visible-pair
    flops), each with its ratio to the NVFP4 paged figure measured the same way."""
    out = []
    for name in ("batch_decode", "asym_decode", "prefill_extend"):
        w = synth.workload(name)
        ref_rate = None
        for dtype, layout in (("nvfp4", "paged"), ("fp8", "paged"), ("nvfp4", "ragged"),
                              ("fp8", "ragged")):
            if layout == "ragged" and w.decode:
                continue
            if layout == "paged":
                cases = [paged.build_case(w, keep_sources=False, dtype=dtype)
                         for _ in range(pool_sets)]
                plan = paged.make_plan(cases[0])
            else:
                cases = [paged.build_ragged_case(w, dtype=dtype) for _ in range(pool_sets)]
                plan = paged.make_ragged_plan(cases[0])
            plan.set_deferred_merge(True)
            ws = plan.new_workspace()
            plan.upload(ws)
            o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim_vo), device="cuda")
            lse = torch.empty((w.total_q, w.num_qo_heads), device="cuda")
            if layout == "ragged":
                run = [nv.batch_prefill_ragged(plan, c.q, c.k, c.v, w.sm_scale, ws, out=o, lse=lse,
                                               prepare=True) for c in cases]
            else:
                fn = nv.batch_decode if w.decode else nv.batch_prefill
                run = [fn(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o,
                          lse=lse, prepare=True) for c in cases]
            merge = nv.merge_partials(plan, ws, o, lse, prepare=True)
            for i in range(warm):
                run[i % len(run)]()
                merge()
            run_ms, merge_ms = timed_passes(torch, nv, run, merge, iters)
            if w.decode:
                q = w.batch * w.num_qo_heads * w.head_dim_qk * 2
                o_b = w.batch * w.num_qo_heads * (w.head_dim_vo * 4 + 4)
                rate = (w.kv_bytes(dtype) + q + o_b) / run_ms / 1e6
                line = {"workload": name, "kv_dtype": dtype, "layout": layout,
                        "kernel_GBs": round(rate, 1),
                        "kernel_frac_hbm": round(rate / HBM_PEAK_GBS, 4),
                        "kv_bytes": w.kv_bytes(dtype)}
            else:
                rate = w.flops() / run_ms / 1e9
                line = {"workload": name, "kv_dtype": dtype, "layout": layout,
                        "kernel_TFLOPs": round(rate, 2),
                        "kernel_frac_mfma_f16": round(rate / MFMA_F16_PEAK_TFLOPS, 4)}
            ref_rate = rate if ref_rate is None else ref_rate
            line.update(attn_ms=round(run_ms, 4), merge_ms=round(merge_ms, 4),
                        vs_nvfp4_paged=round(rate / ref_rate, 4))
            out.append(line)
            del run, merge, cases, ws
            torch.cuda.empty_cache()
    return out


def prefix_masks(w):
    """Multimodal-prefix masks of a prefill workload: the first third of each request's
    new tokens (an image) attend to each other bidirectionally, every row also sees the
    cached prefix and, causally, the tokens up to itself."""
    out = []
    for q, L in zip(w.qo_lens, w.kv_lens):
        prefix, img = L - q, max(1, q // 3)
        i = np.arange(q)[:, None]
        j = np.arange(L)[None, :]
        out.append((j <= i + prefix) | ((i < img) & (j >= prefix) & (j < prefix + img)))
    return out


def masked_prefill_line(torch, nv, paged, synth, iters=60, warm=12, pool_sets=3):
    """The prefill extend under multimodal-prefix masks (nvfp4_batch_prefill_masked),
    beside the same workload's causal run measured the same way.  Flops count the
    pairs the mask leaves visible."""
    w = synth.workload("prefill_extend")
    masks = prefix_masks(w)
    packed = np.concatenate([np.packbits(m.ravel(), bitorder="little") for m in masks] +
                            [np.zeros(8, dtype=np.uint8)])
    visible = int(sum(int(m.sum()) for m in masks))
    flops = 2 * (w.head_dim_qk + w.head_dim_vo) * w.num_qo_heads * visible
    cases = [paged.build_case(w, keep_sources=False) for _ in range(pool_sets)]
    out = {"workload": w.name, "mask": "first third of each request's new tokens "
           "bidirectional, the rest causal", "visible_pairs_per_head": visible,
           "causal_pairs_per_head": w.unmasked_pairs(), "flops": flops}
    for label, custom in (("causal", False), ("masked", True)):
        plan = nv.Plan(w.kv_lens, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                       head_dim_qk=w.head_dim_qk, head_dim_vo=w.head_dim_vo,
                       qo_indptr=cases[0].qo_indptr.tolist(), causal=True, custom_mask=custom)
        plan.set_deferred_merge(True)
        ws = plan.new_workspace()
        plan.upload(ws)
        o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim_vo), device="cuda")
        lse = torch.empty((w.total_q, w.num_qo_heads), device="cuda")
        if custom:
            mask = torch.from_numpy(packed).cuda()
            run = [nv.batch_prefill_masked(plan, c.q, c.page_table, c.k_pool, c.v_pool, mask,
                                           w.sm_scale, ws, out=o, lse=lse, prepare=True)
                   for c in cases]
        else:
            run = [nv.batch_prefill(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws,
                                    out=o, lse=lse, prepare=True) for c in cases]
        merge = nv.merge_partials(plan, ws, o, lse, prepare=True)
        for i in range(warm):
            run[i % len(run)]()
            merge()
        run_ms, merge_ms = timed_passes(torch, nv, run, merge, iters)
        fl = flops if custom else w.flops()
        out[label] = {"kernel_TFLOPs": round(fl / run_ms / 1e9, 2),
                      "kernel_frac_mfma_f16": round(fl / run_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
                      "attn_ms": round(run_ms, 4), "merge_ms": round(merge_ms, 4),
                      "work_items": plan.info()["num_work_items"]}
        del run, merge, ws
    del cases
    torch.cuda.empty_cache()
    return out


def rope_prefill_lines(torch, nv, paged, synth, iters=40, warm=10, pool_sets=3):
    """Prefill with in-kernel RoPE (base 1e4) beside the same workload without it, both
    measured the same way; flops count the QK and PV products of the visible pairs only
    (the rotations are extra vector work on the same pairs)."""
    out = []
    for name in ("prefill_extend", "asym_prefill"):
        w = synth.workload(name)
        cases = [paged.build_case(w, keep_sources=False) for _ in range(pool_sets)]
        line = {"workload": name, "rope_theta": 1e4, "flops": w.flops()}
        for label, rope in (("plain", None), ("rope", (1e4, 1.0))):
            plan = paged.make_plan(cases[0], rope=rope)
            plan.set_deferred_merge(True)
            ws = plan.new_workspace()
            plan.upload(ws)
            o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim_vo), device="cuda")
            lse = torch.empty((w.total_q, w.num_qo_heads), device="cuda")
            run = [nv.batch_prefill(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws,
                                    out=o, lse=lse, prepare=True) for c in cases]
            merge = nv.merge_partials(plan, ws, o, lse, prepare=True)
            for i in range(warm):
                run[i % len(run)]()
                merge()
            run_ms, merge_ms = timed_passes(torch, nv, run, merge, iters)
            rate = w.flops() / run_ms / 1e9
            line[label] = {"kernel_TFLOPs": round(rate, 2),
                           "kernel_frac_mfma_f16": round(rate / MFMA_F16_PEAK_TFLOPS, 4),
                           "attn_ms": round(run_ms, 4), "merge_ms": round(merge_ms, 4)}
            del run, merge, ws
        line["rope_vs_plain"] = round(line["plain"]["attn_ms"] / line["rope"]["attn_ms"], 4)
        out.append(line)
        del cases
        torch.cuda.empty_cache()
    return out


def stream_ceiling(torch, nv, plan, cases, ws, iters, kv_bytes, attn_ms):
    """What the decode access pattern sustains without the attention arithmetic: the
    checksum kernel (nvfp4_kv_checksum) streams the same plan's KV bytes through the same
    rings and copies; timed like the attention kernel (events carried by its dispatch),
    over the same rotated pool sets."""
    w = cases[0].w
    out = torch.empty((w.batch, w.num_kv_heads), dtype=torch.int32, device="cuda")
    calls = [nv.kv_checksum(plan, c.page_table, c.k_pool, c.v_pool, ws, out=out, prepare=True)
             for c in cases]
    for i in range(10):
        calls[i % len(calls)]()
    he = HipEvents()
    ev = [(he.new(), he.new()) for _ in range(iters)]
    for i, (a, b) in enumerate(ev):
        he.time_launches(nv, a, b)
        calls[i % len(calls)]()
        he.time_launches(nv, None, None)
    torch.cuda.synchronize()
    ms = float(np.mean([he.ms(a, b) for a, b in ev]))
    gbs = kv_bytes / ms / 1e6
    return {"kernel": "kv_checksum_kernel", "ms": round(ms, 5), "kv_GBs": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "attention_kernel_vs_ceiling": round(ms / attn_ms, 4)}


def single_decode_latency(torch, nv, paged, synth, iters=300, warm=50):
    """Latency of one single-request decode step (the 128-key, 4/1-head workload):
    the kernel's own duration (events carried by its dispatch) and the host's time from
    the call to the GPU's completion (launch + synchronize), as percentiles in us."""
    w = synth.workload("single_decode")
    case = paged.build_case(w, keep_sources=False)
    plan = paged.make_plan(case)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.empty((w.batch, w.num_qo_heads, w.head_dim_vo), device="cuda")
    lse = torch.empty((w.batch, w.num_qo_heads), device="cuda")
    run = nv.batch_decode(plan, case.q, case.page_table, case.k_pool, case.v_pool, w.sm_scale,
                          ws, out=o, lse=lse, prepare=True)
    for _ in range(warm):
        run()
    torch.cuda.synchronize()
    he = HipEvents()
    ev = [(he.new(), he.new()) for _ in range(iters)]
    wall = []
    for a, b in ev:
        t0 = time.perf_counter()
        he.time_launches(nv, a, b)
        run()
        he.time_launches(nv, None, None)
        torch.cuda.synchronize()
        wall.append((time.perf_counter() - t0) * 1e6)
    kern = [he.ms(a, b) * 1e3 for a, b in ev]

    def pct(x):
        return {f"p{p}": round(float(np.percentile(x, p)), 2) for p in (10, 50, 90)}
    return {"workload": w.name, "kernel_us": pct(kern), "call_to_done_us": pct(wall),
            "iters": iters, "work_items": plan.info()["num_work_items"]}


class Decoder:
    """The timed decode step of one workload over rotated pool sets."""

    def __init__(self, torch, nv, paged, synth, name, pool_sets):
        self.torch, self.nv = torch, nv
        w = self.w = synth.workload(name)
        if not w.decode:
            raise SystemExit("the timed step is a decode workload; prefill runs as an extra line")
        self.sets = [paged.build_case(w, keep_sources=(i == 0)) for i in range(pool_sets)]
        t0 = time.perf_counter()
        self.plan = paged.make_plan(self.sets[0])
        self.plan_us = (time.perf_counter() - t0) * 1e6
        self.plan.set_deferred_merge(True)
        self.ws = self.plan.new_workspace()
        self.plan.upload(self.ws)
        # the step's new token of every request: its K/V rows and the slot of token L_b - 1
        g = torch.Generator(device="cuda")
        g.manual_seed(w.value_seed + 500)
        self.new_k = torch.randn((w.batch, w.num_kv_heads, w.head_dim_qk), generator=g,
                                 device="cuda").bfloat16()
        self.new_v = torch.randn((w.batch, w.num_kv_heads, w.head_dim_vo), generator=g,
                                 device="cuda").bfloat16()
        last = np.cumsum(w.kv_lens) - 1
        self.new_slots = self.sets[0].slots[torch.tensor(last, device="cuda")]
        self.o = torch.empty((w.batch, w.num_qo_heads, w.head_dim_vo), device="cuda")
        self.lse = torch.empty((w.batch, w.num_qo_heads), device="cuda")
        # the two calls of a step (append + attention in one launch, then the merge of the
        # split rows), marshalled once per pool set
        self.calls = [(nv.batch_decode_append(self.plan, c.q, self.new_k, self.new_v,
                                              c.page_table, c.k_pool, c.v_pool, w.sm_scale,
                                              self.ws, out=self.o, lse=self.lse, prepare=True),
                       nv.merge_partials(self.plan, self.ws, self.o, self.lse, prepare=True))
                      for c in self.sets]
        # the same step with a separate append launch (for the breakdown line)
        self.unfused = [(nv.quantize_kv(self.new_k, self.new_v, self.new_slots, c.k_pool,
                                        c.v_pool, prepare=True),
                         nv.batch_decode(self.plan, c.q, c.page_table, c.k_pool, c.v_pool,
                                         w.sm_scale, self.ws, out=self.o, lse=self.lse,
                                         prepare=True),
                         nv.merge_partials(self.plan, self.ws, self.o, self.lse, prepare=True))
                        for c in self.sets]

    def step(self, i, ev=None, he=None):
        """One step; with ``ev`` (two events) the attention launch carries them: the
        dispatch timestamps the kernel's start and end, adding no packet to the queue."""
        attn, merge = self.calls[i % len(self.calls)]
        if ev is None:
            attn()
            merge()
            return
        he.time_launches(self.nv, ev[0], ev[1])
        attn()
        he.time_launches(self.nv, None, None)
        merge()

    def merge_ms(self, iters):
        """Mean duration of the merge launch (outside the timed steps)."""
        s = self.torch.cuda.current_stream()
        he = HipEvents()
        ev = [(he.new(), he.new()) for _ in range(iters)]
        for i, (a, b) in enumerate(ev):
            attn, merge = self.calls[i % len(self.calls)]
            attn()
            he.record(a, s)
            merge()
            he.record(b, s)
        self.torch.cuda.synchronize()
        return float(np.mean([he.ms(a, b) for a, b in ev]))

    def unfused_step_ms(self, iters):
        """Mean GPU time of the step with the append as its own launch."""
        s = self.torch.cuda.current_stream()
        he = HipEvents()
        ev = [(he.new(), he.new()) for _ in range(iters)]
        for i, (a, b) in enumerate(ev):
            quant, attn, merge = self.unfused[i % len(self.unfused)]
            he.record(a, s)
            quant()
            attn()
            merge()
            he.record(b, s)
        self.torch.cuda.synchronize()
        return float(np.mean([he.ms(a, b) for a, b in ev]))


def synth_module():
    """The input-recipe module (no torch device work), for the summaries."""
    sys.path.insert(0, ROOT)
    from attention_bit_paged_amd import synth
    return synth


def pmc_run(args):
    """Short program for counter passes: calibration copy, then a few decode steps."""
    import torch
    import attention_bit_paged_amd as nv
    from attention_bit_paged_amd import paged, synth
    x = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    del x, y
    if args.variant:
        w, case, plan = variant_case(paged, synth, args.workload, args.variant)
        ws = plan.new_workspace()
        plan.upload(ws)
        o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim_vo), device="cuda")
        lse = torch.empty((w.total_q, w.num_qo_heads), device="cuda")
        for _ in range(5):
            nv.batch_decode(plan, case.q, case.page_table, case.k_pool, case.v_pool, w.sm_scale,
                            ws, out=o, lse=lse)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_run": args.workload, "variant": args.variant,
                          "info": plan.info()}), flush=True)
        return
    d = Decoder(torch, nv, paged, synth, args.workload, 1)
    for i in range(5):
        d.step(i)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_run": args.workload, "info": d.plan.info()}), flush=True)


def _kernel_rows(path_glob):
    files = glob.glob(path_glob, recursive=True)
    if not files:
        raise SystemExit(f"no file matches {path_glob}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _short(name):
    name = name.replace("void ", "").replace("nvfp4::(anonymous namespace)::", "")
    return name.split("(")[0][:70]


def summarize_trace(args):
    rows = _kernel_rows(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel trace summary, workload {args.workload}",
             f"# command: {args.command}", "",
             f"{'kernel':72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{_short(r['Name']):72s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} "
                     f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} "
                     f"{float(r['Percentage']):6.2f}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def summarize_pmc(args):
    """FETCH_SIZE / WRITE_SIZE per dispatch of the decode kernel and of the 1 GiB copy
    (its calibration), into the traffic record the benchmark reads back."""
    fetch_dir, write_dir = args.summarize_pmc

    def per_kernel(d, counter):
        out = {}
        rows = _kernel_rows(os.path.join(d, "**", "*counter_collection.csv"))
        for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    # the decode launch with the append (the benchmark's step), else the plain decode
    # kernel of a --variant run
    dec = ([k for k in fetch if "decode_ring_kernel" in k and "true" in k] or
           [k for k in fetch if "decode_ring_kernel" in k or "decode_regs_kernel" in k])
    cpy = [k for k in fetch if "copyBuffer" in k]
    if not dec or not cpy:
        raise SystemExit(f"kernels not found: {list(fetch)}")
    # --pmc-run starts with three copies of CALIB_BYTES: the first three copy dispatches
    dk, ck = dec[0], cpy[0]
    kib = CALIB_BYTES / 1024
    f_scale = kib / float(np.mean(fetch[ck][:3]))
    w_scale = kib / float(np.mean(write[ck][:3]))
    f_dec, w_dec = float(np.mean(fetch[dk])), float(np.mean(write[dk]))
    nbytes = (f_dec * f_scale + w_dec * w_scale) * 1024
    variant = getattr(args, "variant", "")
    if variant:
        w = variant_workload(synth_module(), args.workload, variant)[0]
        kv, qo = decode_bytes(w)
    else:
        kv, qo = decode_bytes(synth_module().workload(args.workload), append=True)
    rec = {"kernel": _short(dk), "workload": args.workload, "variant": variant or None,
           "algorithmic_bytes": kv + qo,
           "fetch_kib_per_dispatch": round(f_dec, 1), "write_kib_per_dispatch": round(w_dec, 1),
           "copy_fetch_kib": round(float(np.mean(fetch[ck][:3])), 1),
           "copy_write_kib": round(float(np.mean(write[ck][:3])), 1),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "bytes_per_launch": round(nbytes),
           "traffic_over_algorithmic": round(nbytes / (kv + qo), 4),
           "source_digest": sources_digest()}
    text = "\n".join([
        f"# HBM traffic of the decode kernel, workload {args.workload}",
        f"# commands: {args.command}",
        f"# calibration: {_short(ck)} copies {CALIB_BYTES} bytes; FETCH_SIZE reads "
        f"{rec['copy_fetch_kib']} KiB and WRITE_SIZE {rec['copy_write_kib']} KiB for it, so the "
        f"scales are {rec['fetch_scale']} and {rec['write_scale']}",
        f"# decode kernel {rec['kernel']}{' (' + variant + ')' if variant else ''}: "
        f"FETCH_SIZE {rec['fetch_kib_per_dispatch']} KiB, "
        f"WRITE_SIZE {rec['write_kib_per_dispatch']} KiB per dispatch "
        f"({len(fetch[dk])} dispatches) -> {rec['bytes_per_launch']} bytes per launch, "
        f"{rec['traffic_over_algorithmic']} x the {rec['algorithmic_bytes']} algorithmic bytes",
        json.dumps(rec)]) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


SIMDS = 256 * 4          # MI355X: 256 CUs of 4 SIMDs
CLOCK_GHZ = 2.4          # nominal peak engine clock (used only without GRBM_GUI_ACTIVE)
XCCS = 8                 # GRBM_GUI_ACTIVE is counted per XCC (dimension XCC[0:7]) and summed


def summarize_counters(args):
    """Per-dispatch SQ counters of one kernel from rocprofv3 --pmc passes, averaged over
    its dispatches, with the figures derived from them.  Cycle counters of waves
    (SQ_WAVE_CYCLES, SQ_WAIT_*, SQ_ACTIVE_INST_*) count in units of 4 cycles;
    SQ_VALU_MFMA_BUSY_CYCLES in cycles, summed over the SIMDs.  Kernel time comes from
    the dispatch timestamps.  The engine clock is measured when a pass holds
    GRBM_GUI_ACTIVE (the cycles the graphics engine was busy, summed over the 8 XCCs:
    clock = GRBM_GUI_ACTIVE / 8 / kernel time), else the nominal 2.4 GHz is assumed;
    rocprofv3's own derived MfmaUtil, when a pass holds it, is reported beside ours."""
    vals, dur, waves = {}, [], None
    for d in args.summarize_counters:
        per = {}
        for r in _kernel_rows(os.path.join(d, "**", "*counter_collection.csv")):
            if args.kernel not in r["Kernel_Name"]:
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            dur.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
            waves = int(r["Grid_Size"]) // 64
        for (_, c), v in per.items():
            vals.setdefault(c, []).append(v)
    if not vals:
        raise SystemExit(f"no dispatch of {args.kernel} in {args.summarize_counters}")
    avg = {c: float(np.mean(v)) for c, v in vals.items()}
    t = float(np.median(dur))
    clock_ghz, clock_src = CLOCK_GHZ, "nominal"
    if avg.get("GRBM_GUI_ACTIVE", 0) > 0:
        clock_ghz, clock_src = avg["GRBM_GUI_ACTIVE"] / XCCS / t / 1e9, "measured"
    cyc = t * clock_ghz * 1e9
    lines = [f"# SQ counters of {args.kernel}, workload {args.workload}",
             f"# command: {args.command}",
             f"# {len(vals[next(iter(vals))])} dispatches per counter; kernel {t * 1e6:.1f} us "
             f"(dispatch timestamps, median), {waves} waves; engine clock {clock_ghz:.3f} GHz "
             f"({clock_src})", ""]
    for c in sorted(avg):
        lines.append(f"{c:32s} {avg[c]:18.0f}")
    der = {"clock_ghz": clock_ghz}
    if "MfmaUtil" in avg:
        der["rocprof_mfma_util_share"] = avg["MfmaUtil"] / 100
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        der["mfma_busy_share"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cyc)
    if "SQ_INSTS_VALU_MFMA_MOPS_F16" in avg:
        der["mfma_f16_tflops_executed"] = avg["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 / t / 1e12
    if "SQ_WAVE_CYCLES" in avg:
        der["resident_wave_share_of_2_per_simd"] = avg["SQ_WAVE_CYCLES"] * 4 / (2 * SIMDS * cyc)
    if "SQ_INSTS_MFMA" in avg and waves:
        mf = avg["SQ_INSTS_MFMA"] / waves
        der["mfma_per_wave"] = mf
        if "SQ_INSTS_VALU" in avg:
            der["other_valu_per_mfma"] = (avg["SQ_INSTS_VALU"] - avg["SQ_INSTS_MFMA"]) / avg["SQ_INSTS_MFMA"]
        for c in ("SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VALU_TRANS_F32"):
            if c in avg:
                der[c.lower() + "_per_mfma"] = avg[c] / avg["SQ_INSTS_MFMA"]
        for c in ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY",
                  "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS"):
            if c in avg:
                der[c.lower() + "_cycles_per_mfma"] = avg[c] * 4 / avg["SQ_INSTS_MFMA"]
    lines += ["", "# derived (per MFMA instruction: 16 busy cycles each for 16x16x32 f16)"]
    lines += [f"{k:48s} {v:12.4f}" for k, v in der.items()]
    lines.append(json.dumps({"kernel": args.kernel, "workload": args.workload, "kernel_us": round(t * 1e6, 2),
                             "clock": clock_src,
                             "counters": {c: round(v) for c, v in avg.items()},
                             "derived": {k: round(v, 4) for k, v in der.items()}}))
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def prefill_main(args, torch, nv, paged, synth):
    """A prefill workload as the timed step (for profiling the prefill kernel): the
    attention pass and the merge of its split rows, prepared once."""
    w = synth.workload(args.workload)
    case = paged.build_case(w, keep_sources=False)
    plan = paged.make_plan(case)
    plan.set_deferred_merge(True)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.empty((w.total_q, w.num_qo_heads, w.head_dim_vo), device="cuda")
    lse = torch.empty((w.total_q, w.num_qo_heads), device="cuda")
    run = nv.batch_prefill(plan, case.q, case.page_table, case.k_pool, case.v_pool, w.sm_scale,
                           ws, out=o, lse=lse, prepare=True)
    merge = nv.merge_partials(plan, ws, o, lse, prepare=True)
    for _ in range(args.warmup):
        run()
        merge()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_ms, merge_ms = timed_passes(torch, nv, run, merge, args.steps)
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    fl = w.flops()
    info = plan.info()
    out = {"metric": "NVFP4 paged prefill TFLOP/s (% MFMA peak)",
           "value": round(fl / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic (seeded N(0,1) bf16 Q/K/V, K/V NVFP4-quantised on the GPU)",
           "config": {"workload": w.name, "batch": w.batch, "num_qo_heads": w.num_qo_heads,
                      "num_kv_heads": w.num_kv_heads, "head_dim_qk": w.head_dim_qk,
                      "head_dim_vo": w.head_dim_vo, "causal": w.causal,
                      "work_items": info["num_work_items"]},
           "roofline": {"bound": "mfma", "achieved": round(fl / run_ms / 1e9, 2),
                        "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(fl / run_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
                        "traffic": None, "flops_per_launch": fl,
                        "avg_launch_ms": round(run_ms, 5)},
           "step_breakdown_ms": {"attention": round(run_ms, 5), "merge": round(merge_ms, 5)}}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by request or kv head with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    if args.pmc_run:
        return pmc_run(args)
    import torch
    import attention_bit_paged_amd as nv
    from attention_bit_paged_amd import paged, synth

    if not synth.workload(args.workload).decode:
        return prefill_main(args, torch, nv, paged, synth)
    d = Decoder(torch, nv, paged, synth, args.workload, args.pool_sets)
    w, info = d.w, d.plan.info()
    for i in range(args.warmup):
        d.step(i)
    torch.cuda.synchronize()
    he = HipEvents()
    ev = [[he.new() for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        d.step(i, ev[i], he)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    launch_ms = np.array([he.ms(e[0], e[1]) for e in ev])
    attn_ms = float(np.mean(launch_ms))
    # breakdown, after the timed steps
    merge_ms = d.merge_ms(max(args.steps // 2, 3))
    unfused_ms = d.unfused_step_ms(max(args.steps // 2, 3))
    kv_only, _ = decode_bytes(w)
    ceiling = stream_ceiling(torch, nv, d.plan, d.sets, d.ws, max(args.steps // 2, 3), kv_only,
                             attn_ms)

    kv, qo = decode_bytes(w, append=True)
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = (kv + qo) / (attn_ms * 1e-3) / 1e9
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
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, K/V NVFP4-quantised on the GPU)",
        "config": {"workload": w.name, "batch": w.batch,
                   "kv_len": (str(w.kv_lens[0]) if min(w.kv_lens) == max(w.kv_lens)
                              else f"{min(w.kv_lens)}..{max(w.kv_lens)} (seeded uniform)"),
                   "num_qo_heads": w.num_qo_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim_qk, "page_size": w.page_size, "pool_pages": w.pool_pages,
                   "kv_chunk_tokens": info["kv_chunk_tokens"],
                   "kv_chunk_tokens_meaning": "keys per wave part; a work item (workgroup of "
                   "four waves) covers four consecutive parts, and split rows are merged per "
                   "work item",
                   "keys_per_work_item": 4 * info["kv_chunk_tokens"],
                   "work_items": info["num_work_items"],
                   "total_kv_tokens": w.total_kv, "pool_sets_rotated": len(d.sets)},
        "frac_hbm": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(w.name),
                     "kernel": f"decode_ring_kernel<{w.head_dim_qk}, {w.head_dim_vo}, true>",
                     "bytes_per_launch": kv + qo, "avg_launch_ms": round(attn_ms, 5)},
        "kernel_ms_percentiles": {"p10": round(float(np.percentile(launch_ms, 10)), 5),
                                  "p50": round(float(np.percentile(launch_ms, 50)), 5),
                                  "p90": round(float(np.percentile(launch_ms, 90)), 5)},
        "step_breakdown_ms": {"append_and_attention": round(attn_ms, 5),
                              "merge": round(merge_ms, 5),
                              "unfused_step_gpu": round(unfused_ms, 5)},
        "plan_host_us": round(d.plan_us, 1),
        "stream_ceiling": ceiling,
    }
    budget = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    if not args.no_cpu_baseline:
        cb = cpu_baseline(d.sets[0], budget, cpu_threads())
        out["cpu_baseline"] = {
            "value": cb["value_threads"], "unit": "GB/s", "cores": cb["threads"], "kind": "oracle",
            "sample": f"{cb['sample_threads']} of the {w.name} workload on {cb['threads']} host "
                      "threads (numpy float64, BLAS one thread each; pairs run in parallel)",
            "value_1_thread": cb["value_1_thread"], "sample_1_thread": cb["sample_1_thread"],
            "full_workload_s_extrapolated": cb["full_workload_s_extrapolated"]}
    if not args.no_extra:
        del d
        torch.cuda.empty_cache()
        out["single_decode_latency"] = single_decode_latency(torch, nv, paged, synth)
        extras = [extra_decode(torch, nv, paged, synth, n, cpu_budget=budget)
                  for n in ("long_decode", "asym_decode")]
        extras += [extra_prefill(torch, nv, paged, synth, n, cpu_budget=budget)
                   for n in ("prefill_extend", "asym_prefill")]
        out["other_workloads"] = extras
        out["layout_variants"] = [variant_lines(torch, nv, paged, synth, n)
                                  for n in ("batch_decode", "prefill_extend")]
        out["kv_types"] = kv_type_lines(torch, nv, paged, synth)
        out["masked_prefill"] = masked_prefill_line(torch, nv, paged, synth)
        out["rope_prefill"] = rope_prefill_lines(torch, nv, paged, synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
