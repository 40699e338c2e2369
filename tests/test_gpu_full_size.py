"""Parity at the benchmark workloads' full sizes, in the launch configuration the
benchmark times (its plans, chunking and entry points), on sampled requests and kv
heads that the oracle computes one by one from the pools' bytes.

The caches are built on the GPU by the append kernel (whose bytes are pinned to the
oracle quantiser by the bit-exact tests); the oracle reads those bytes back, so these
tests check the attention path itself at full size: page tables of tens of thousands
of pages, split-KV with the benchmark's chunking, and the merge."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import paged, synth
from oracle import nvfp4_ref as ref
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _oracle_rows(case, o, lse, samples, causal=False):
    """Compare O/LSE of the sampled (request, kv head) pairs with the oracle."""
    w = case.w
    kd, ks = case.k_pool.data.cpu().numpy(), case.k_pool.sf.cpu().numpy()
    vd, vs = case.v_pool.data.cpu().numpy(), case.v_pool.sf.cpu().numpy()
    q = case.q.float().cpu().double().numpy()
    g = w.group
    ind = synth.indptr(w.qo_lens)
    for b, h in samples:
        q0, q1 = int(ind[b]), int(ind[b + 1])
        qs = q[:, g * h:g * (h + 1)]
        o_ref, lse_ref = ref.paged_attention(
            qs, kd[:, h:h + 1], ks[:, h:h + 1], vd[:, h:h + 1], vs[:, h:h + 1],
            case.page_table_np, w.kv_lens, ind, w.page_size, w.sm_scale, causal, "HND",
            rows=[b])
        gh.assert_attention_close(o[q0:q1, g * h:g * (h + 1)], lse[q0:q1, g * h:g * (h + 1)],
                                  o_ref[q0:q1], lse_ref[q0:q1], f"{w.name} b={b} h={h}")


def _decode(name, fused):
    w = synth.workload(name)
    case = paged.build_case(w, keep_sources=False)
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


def test_batch_decode_full_size_with_append():
    """64 requests of 543..7978 keys, 256-key chunks, the step's token appended in the
    launch: the shortest, a middle and the longest request, two kv heads each."""
    case, o, lse = _decode("batch_decode", fused=True)
    lens = np.array(case.w.kv_lens)
    picks = [int(np.argmin(lens)), 31, int(np.argmax(lens))]
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_rows(case, o, lse, [(b, h) for b in picks for h in (0, 7)])


def test_long_decode_full_size():
    """8 requests of 131072 keys, split to fill the device."""
    case, o, lse = _decode("long_decode", fused=False)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_rows(case, o, lse, [(2, 5)])


def test_asym_decode_full_size():
    """32 requests of 32768 keys, head dims 512/256, 8 qo heads on one kv head."""
    case, o, lse = _decode("asym_decode", fused=False)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _oracle_rows(case, o, lse, [(0, 0), (19, 0)])


def test_prefill_extend_full_size():
    """16 requests, causal extend over prefixes of 0..4096 keys: two requests, one kv
    head each."""
    w = synth.workload("prefill_extend")
    case = paged.build_case(w, keep_sources=False)
    plan = paged.make_plan(case)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.full((w.total_q, w.num_qo_heads, w.head_dim_vo), float("nan"), device="cuda")
    lse = torch.full((w.total_q, w.num_qo_heads), float("nan"), device="cuda")
    nv.batch_prefill(plan, case.q, case.page_table, case.k_pool, case.v_pool, w.sm_scale, ws,
                     out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    lens = np.array(w.kv_lens)
    _oracle_rows(case, o, lse, [(int(np.argmax(lens)), 3), (int(np.argmin(lens)), 6)],
                 causal=True)
