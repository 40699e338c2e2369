"""Parity at the benchmark workloads' full sizes, in the launch configuration the
benchmark times (its plans, chunking and entry points), on a seeded random quarter of
the (request, kv head) pairs that the oracle computes one by one from the pools' bytes.
The shortest and the longest request are always in the sample.

The caches are built on the GPU by the append kernel (whose bytes are pinned to the
oracle quantiser by the bit-exact tests); the oracle reads those bytes back, so these
tests check the attention path itself at full size: page tables of tens of thousands
of pages, split-KV with the benchmark's chunking, and the merge.  Every pair's largest
O error and LSE error are asserted and recorded (``record_property``; a junit XML run
keeps them)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import paged, synth
from oracle import nvfp4_ref as ref
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

SAMPLE_FRACTION = 0.25


def sample_pairs(w: synth.Workload, seed: int, frac: float = SAMPLE_FRACTION):
    """A seeded random ``frac`` of the (request, kv head) pairs, plus one pair of the
    shortest and one of the longest request when the draw missed them."""
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    rng = np.random.default_rng(seed)
    n = max(1, math.ceil(frac * len(pairs)))
    pick = {pairs[i] for i in rng.choice(len(pairs), size=n, replace=False)}
    lens = np.asarray(w.kv_lens)
    for b in (int(np.argmin(lens)), int(np.argmax(lens))):
        if not any(p[0] == b for p in pick):
            pick.add((b, int(rng.integers(w.num_kv_heads))))
    return sorted(pick)


def _oracle_pairs(case, o, lse, samples, record, causal=False, rope=None):
    """Compare O/LSE of the sampled (request, kv head) pairs with the oracle; returns
    the largest O error over them."""
    w = case.w
    host = lambda t: None if t is None else t.cpu().numpy()
    kd, ks = host(case.k_pool.data), host(case.k_pool.sf)
    vd, vs = host(case.v_pool.data), host(case.v_pool.sf)
    head = lambda a, h: None if a is None else a[:, h:h + 1]
    q = case.q.float().cpu().double().numpy()
    g = w.group
    ind = synth.indptr(w.qo_lens)
    worst, errs = 0.0, {}
    for b, h in samples:
        q0, q1 = int(ind[b]), int(ind[b + 1])
        qs = q[:, g * h:g * (h + 1)]
        o_ref, lse_ref = ref.paged_attention(
            qs, head(kd, h), head(ks, h), head(vd, h), head(vs, h),
            case.page_table_np, w.kv_lens, ind, w.page_size, w.sm_scale, causal, "HND",
            rows=[b], kv_dtype=case.k_pool.dtype, rope=rope)
        og, lg = o[q0:q1, g * h:g * (h + 1)], lse[q0:q1, g * h:g * (h + 1)]
        err = gh.assert_attention_close(og, lg, o_ref[q0:q1], lse_ref[q0:q1],
                                        f"{w.name} b={b} h={h}")
        lerr = float((np.abs(lg - lse_ref[q0:q1]) / np.maximum(1.0, np.abs(lse_ref[q0:q1]))).max())
        errs[f"b{b}_h{h}"] = (round(float(err), 7), round(lerr, 9))
        worst = max(worst, float(err))
    record("pairs_checked", len(samples))
    record("pairs_total", w.batch * w.num_kv_heads)
    record("max_abs_err_O", worst)
    record("per_pair_O_err_LSE_relerr", errs)
    print(f"{w.name}: {len(samples)} of {w.batch * w.num_kv_heads} (request, kv head) pairs, "
          f"max |O err| {worst:.3e}", flush=True)
    return worst


def _decode(name, fused, dtype="nvfp4"):
    w = synth.workload(name)
    case = paged.build_case(w, keep_sources=False, dtype=dtype)
    plan = paged.make_plan(case)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.full((w.batch, w.num_qo_heads, w.head_dim_vo), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.num_qo_heads), float("nan"), device="cuda")
    if fused:
        g = torch.Generator(device="cuda")
        g.manual_seed(w.value_seed + 500)
        kn = torch.randn((w.batch, w.num_kv_heads, w.head_dim_qk), generator=g, device="cuda")
        vn = torch.randn((w.batch, w.num_kv_heads, w.head_dim_vo), generator=g, device="cuda")
        nv.batch_decode_append(plan, case.q, kn.bfloat16(), vn.bfloat16(), case.page_table,
                               case.k_pool, case.v_pool, w.sm_scale, ws, out=o, lse=lse)
    else:
        nv.batch_decode(plan, case.q, case.page_table, case.k_pool, case.v_pool, w.sm_scale, ws,
                        out=o, lse=lse)
    torch.cuda.synchronize()
    return case, o.cpu().double().numpy(), lse.cpu().double().numpy()


def _prefill(name, dtype="nvfp4", rope=None):
    w = synth.workload(name)
    case = paged.build_case(w, keep_sources=False, dtype=dtype)
    plan = paged.make_plan(case, rope=rope)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.full((w.total_q, w.num_qo_heads, w.head_dim_vo), float("nan"), device="cuda")
    lse = torch.full((w.total_q, w.num_qo_heads), float("nan"), device="cuda")
    nv.batch_prefill(plan, case.q, case.page_table, case.k_pool, case.v_pool, w.sm_scale, ws,
                     out=o, lse=lse)
    torch.cuda.synchronize()
    return case, o.cpu().double().numpy(), lse.cpu().double().numpy()


@pytest.mark.timeout(600)
def test_batch_decode_full_size_with_append(record_property):
    """64 requests of 543..7978 keys, 256-key chunks, the step's token appended in the
    launch."""
    case, o, lse = _decode("batch_decode", fused=True)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 52), record_property)


@pytest.mark.timeout(600)
def test_long_decode_full_size(record_property):
    """8 requests of 131072 keys, split to fill the device."""
    case, o, lse = _decode("long_decode", fused=False)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 53), record_property)


@pytest.mark.timeout(600)
def test_asym_decode_full_size(record_property):
    """32 requests of 32768 keys, head dims 512/256, 8 qo heads on one kv head."""
    case, o, lse = _decode("asym_decode", fused=False)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 56), record_property)


@pytest.mark.timeout(600)
def test_prefill_extend_full_size(record_property):
    """16 requests, causal extend over prefixes of 0..4096 keys."""
    case, o, lse = _prefill("prefill_extend")
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 54), record_property, causal=True)


@pytest.mark.timeout(600)
def test_asym_prefill_full_size(record_property):
    """4 causal requests of 1024 queries, head dims 512/256: every pair."""
    case, o, lse = _prefill("asym_prefill")
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 55, frac=1.0), record_property, causal=True)


@pytest.mark.timeout(600)
def test_batch_decode_full_size_fp8(record_property):
    """The batch decode workload over an FP8 cache (quantised on the GPU by the FP8
    append kernel, whose bytes are pinned to the oracle by the bit-exact test)."""
    case, o, lse = _decode("batch_decode", fused=False, dtype="fp8")
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 57), record_property)


@pytest.mark.timeout(600)
def test_prefill_extend_full_size_fp8(record_property):
    case, o, lse = _prefill("prefill_extend", dtype="fp8")
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 58), record_property, causal=True)


@pytest.mark.timeout(600)
def test_asym_decode_full_size_fp8(record_property):
    """The 512/256 decode workload over an FP8 cache (the per-token register kernel)."""
    case, o, lse = _decode("asym_decode", fused=False, dtype="fp8")
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 61), record_property)


@pytest.mark.timeout(600)
def test_prefill_extend_full_size_rope(record_property):
    """The prefill extend with in-kernel RoPE (base 1e4), in the benchmark's launch."""
    case, o, lse = _prefill("prefill_extend", rope=(1e4, 1.0))
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 59), record_property, causal=True,
                  rope=(1e4, 1.0))


@pytest.mark.timeout(600)
def test_asym_prefill_full_size_rope(record_property):
    """4 causal requests of 1024 queries, head dims 512/256, RoPE over the 512-dim QK
    rows: every pair."""
    case, o, lse = _prefill("asym_prefill", rope=(1e4, 1.0))
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_pairs(case, o, lse, sample_pairs(case.w, 60, frac=1.0), record_property, causal=True,
                  rope=(1e4, 1.0))


def _prefix_masks(w):
    """The benchmark's multimodal-prefix masks: the first third of each request's new
    tokens attend to each other bidirectionally, the rest causal over the prefix."""
    out = []
    for q, L in zip(w.qo_lens, w.kv_lens):
        prefix, img = L - q, max(1, q // 3)
        i = np.arange(q)[:, None]
        j = np.arange(L)[None, :]
        out.append((j <= i + prefix) | ((i < img) & (j >= prefix) & (j < prefix + img)))
    return out


@pytest.mark.timeout(600)
def test_prefill_extend_full_size_masked(record_property):
    """The prefill extend under the benchmark's multimodal-prefix masks, in its launch
    (nvfp4_batch_prefill_masked, whole-key-range tiles)."""
    w = synth.workload("prefill_extend")
    case = paged.build_case(w, keep_sources=False)
    plan = nv.Plan(w.kv_lens, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                   head_dim_qk=w.head_dim_qk, head_dim_vo=w.head_dim_vo,
                   qo_indptr=case.qo_indptr.tolist(), causal=True, custom_mask=True)
    packed = ref.pack_masks(_prefix_masks(w))
    assert packed.size == plan.mask_bytes
    mask = torch.from_numpy(np.concatenate([packed, np.full(8, 0xFF, np.uint8)])).cuda()
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.full((w.total_q, w.num_qo_heads, w.head_dim_vo), float("nan"), device="cuda")
    lse = torch.full((w.total_q, w.num_qo_heads), float("nan"), device="cuda")
    nv.batch_prefill_masked(plan, case.q, case.page_table, case.k_pool, case.v_pool, mask,
                            w.sm_scale, ws, out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    host = lambda t: None if t is None else t.cpu().numpy()
    kd, ks, vd, vs = (host(case.k_pool.data), host(case.k_pool.sf), host(case.v_pool.data),
                      host(case.v_pool.sf))
    q = case.q.float().cpu().double().numpy()
    g, ind = w.group, synth.indptr(w.qo_lens)
    worst = 0.0
    samples = sample_pairs(w, 61)
    for b, h in samples:
        q0, q1 = int(ind[b]), int(ind[b + 1])
        o_ref, lse_ref = ref.paged_attention(
            q[:, g * h:g * (h + 1)], kd[:, h:h + 1], ks[:, h:h + 1], vd[:, h:h + 1],
            vs[:, h:h + 1], case.page_table_np, w.kv_lens, ind, w.page_size, w.sm_scale, False,
            "HND", rows=[b], custom_mask=packed)
        err = gh.assert_attention_close(o[q0:q1, g * h:g * (h + 1)], lse[q0:q1, g * h:g * (h + 1)],
                                        o_ref[q0:q1], lse_ref[q0:q1], f"masked b={b} h={h}")
        worst = max(worst, float(err))
    record_property("pairs_checked", len(samples))
    record_property("max_abs_err_O", worst)
    print(f"masked prefill_extend: {len(samples)} pairs, max |O err| {worst:.3e}", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["nvfp4", "fp8"])
def test_prefill_extend_full_size_ragged(dtype, record_property):
    """The prefill extend over ragged (non-paged) rows, in the benchmark's launch."""
    w = synth.workload("prefill_extend")
    case = paged.build_ragged_case(w, dtype=dtype)
    plan = paged.make_ragged_plan(case)
    ws = plan.new_workspace()
    plan.upload(ws)
    o, lse = nv.batch_prefill_ragged(plan, case.q, case.k, case.v, w.sm_scale, ws)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    host = lambda t: None if t is None else t.cpu().numpy()
    kd, ks, vd, vs = host(case.k.data), host(case.k.sf), host(case.v.data), host(case.v.sf)
    q = case.q.float().cpu().double().numpy()
    g, ind = w.group, synth.indptr(w.qo_lens)
    worst = 0.0
    samples = sample_pairs(w, 62)
    head = lambda a, h: None if a is None else a[:, h:h + 1]
    for b, h in samples:
        q0, q1 = int(ind[b]), int(ind[b + 1])
        a0, a1 = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        o_ref, lse_ref = ref.ragged_attention(
            q[q0:q1, g * h:g * (h + 1)], head(kd, h)[a0:a1], None if ks is None else
            head(ks, h)[a0:a1], head(vd, h)[a0:a1], None if vs is None else head(vs, h)[a0:a1],
            [0, a1 - a0], [0, q1 - q0], w.sm_scale, True, kv_dtype=dtype)
        err = gh.assert_attention_close(o[q0:q1, g * h:g * (h + 1)], lse[q0:q1, g * h:g * (h + 1)],
                                        o_ref, lse_ref, f"ragged {dtype} b={b} h={h}")
        worst = max(worst, float(err))
    record_property("pairs_checked", len(samples))
    record_property("max_abs_err_O", worst)
    print(f"ragged {dtype} prefill_extend: {len(samples)} pairs, max |O err| {worst:.3e}",
          flush=True)
