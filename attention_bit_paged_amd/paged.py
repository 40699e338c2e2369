"""Device-side set-up of a paged NVFP4 cache for a synthetic workload.

Draws the workload's Q/K/V on the device, allocates separate K and V pools (with
their scale pools) in the requested layout, fills every slot with random bytes and
NaN scales, then writes each request's tokens with ``quantize_kv``.  Used by the
benchmark and by the full-size tests.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import KVPool, Plan, RaggedKV, quantize_kv, synth


@dataclasses.dataclass
class PagedCase:
    w: synth.Workload
    q: torch.Tensor
    k: torch.Tensor          # bf16 source rows (kept for sampling by tests)
    v: torch.Tensor
    k_pool: KVPool
    v_pool: KVPool
    page_table: torch.Tensor
    page_table_np: np.ndarray
    slots: torch.Tensor
    qo_indptr: np.ndarray


def poison_pool(pool: KVPool, seed: int) -> None:
    g = torch.Generator(device=pool.data.device)
    g.manual_seed(seed)
    pool.data.copy_(torch.randint(0, 256, tuple(pool.data.shape), generator=g, dtype=torch.uint8,
                                  device=pool.data.device))
    if pool.sf is not None:
        pool.sf.fill_(synth.SF_POISON)


def padded_pool(w: synth.Workload, head_dim: int, layout: str, device, pad,
                dtype: str = "nvfp4") -> KVPool:
    """A pool whose tensors are views into larger parents, so that its strides differ
    from a dense pool's: ``pad`` = extra (pages, heads, tokens, bytes per row) of the
    parent (the scale rows get 8 extra bytes when the data rows get any)."""
    pp, ph, pt, pb = pad
    H, P = w.num_kv_heads, w.page_size
    if layout == "HND":
        lead, view = (w.pool_pages + pp, H + ph, P + pt), (w.pool_pages, H, P)
    else:
        lead, view = (w.pool_pages + pp, P + pt, H + ph), (w.pool_pages, P, H)
    row = head_dim if dtype == "fp8" else head_dim // 2
    data = torch.empty(lead + (row + pb,), dtype=torch.uint8, device=device)
    idx = tuple(slice(0, n) for n in view)
    sf = None
    if dtype != "fp8":
        sf = torch.empty(lead + (head_dim // 16 + (8 if pb else 0),), dtype=torch.uint8,
                         device=device)[idx + (slice(0, head_dim // 16),)]
    return KVPool(data[idx + (slice(0, row),)], sf, head_dim=head_dim, layout=layout, dtype=dtype)


def build_case(w: synth.Workload, device="cuda", layout="HND", poison=True,
               keep_sources=True, k_pad=None, v_pad=None, dtype: str = "nvfp4") -> PagedCase:
    """``k_pad`` / ``v_pad``: give that pool padded parents (see ``padded_pool``);
    ``dtype``: the pools' KV type ("nvfp4" or "fp8")."""
    q, k, v = synth.draw_qkv(w, device=device)
    if k_pad is None:
        k_pool = KVPool.empty(w.pool_pages, w.num_kv_heads, w.page_size, w.head_dim_qk, layout,
                              device, dtype=dtype)
    else:
        k_pool = padded_pool(w, w.head_dim_qk, layout, device, k_pad, dtype)
    if v_pad is None:
        v_pool = KVPool.empty(w.pool_pages, w.num_kv_heads, w.page_size, w.head_dim_vo, layout,
                              device, dtype=dtype)
    else:
        v_pool = padded_pool(w, w.head_dim_vo, layout, device, v_pad, dtype)
    if poison:
        poison_pool(k_pool, w.value_seed + 11)
        poison_pool(v_pool, w.value_seed + 12)
    pt = synth.page_table(w)
    slots = torch.from_numpy(synth.token_slots(w, pt)).to(device)
    quantize_kv(k, v, slots, k_pool, v_pool)
    ind = synth.indptr(w.qo_lens)
    if not keep_sources:
        k = v = None
    return PagedCase(w, q, k, v, k_pool, v_pool, torch.from_numpy(pt).to(device), pt, slots, ind)


def make_plan(case: PagedCase, num_cus: int = 0, kv_chunk_tokens: Optional[int] = None,
              rope: Optional[tuple] = None) -> Plan:
    """The case's plan; ``rope`` = (theta, scale) turns on the in-kernel rotary (prefill)."""
    w = case.w
    chunk = w.kv_chunk_tokens if kv_chunk_tokens is None else kv_chunk_tokens
    theta, scale = rope if rope is not None else (None, 1.0)
    return Plan(w.kv_lens, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                head_dim_qk=w.head_dim_qk, head_dim_vo=w.head_dim_vo, page_size=w.page_size,
                qo_indptr=None if w.decode else case.qo_indptr.tolist(), causal=w.causal,
                kv_chunk_tokens=chunk, num_cus=num_cus, kv_dtype=case.k_pool.dtype,
                rope_theta=theta, rope_scale=scale)


@dataclasses.dataclass
class RaggedCase:
    w: synth.Workload
    q: torch.Tensor
    k: RaggedKV
    v: RaggedKV
    kv_indptr: np.ndarray
    qo_indptr: np.ndarray


def build_ragged_case(w: synth.Workload, device="cuda", dtype: str = "nvfp4",
                      start: int = 0) -> RaggedCase:
    """The workload's K/V as ragged rows (requests back to back from row ``start``),
    quantised by ``quantize_kv`` through a one-row-per-page view of the same tensors;
    the rows around them hold random bytes (and NaN scales)."""
    q, k, v = synth.draw_qkv(w, device=device)
    rows = []
    for x, d, seed in ((k, w.head_dim_qk, 21), (v, w.head_dim_vo, 22)):
        r = RaggedKV.empty(start + w.total_kv, w.num_kv_heads, d, device=device, dtype=dtype)
        g = torch.Generator(device=r.data.device)
        g.manual_seed(w.value_seed + seed)
        r.data.copy_(torch.randint(0, 256, tuple(r.data.shape), generator=g, dtype=torch.uint8,
                                   device=r.data.device))
        if r.sf is not None:
            r.sf.fill_(synth.SF_POISON)
        rows.append(r)
    views = [KVPool(r.data.unsqueeze(2), None if r.sf is None else r.sf.unsqueeze(2),
                    head_dim=r.head_dim, layout="HND", dtype=dtype) for r in rows]
    slots = torch.arange(start, start + w.total_kv, dtype=torch.int64, device=q.device)
    quantize_kv(k, v, slots, views[0], views[1])
    kv_ind = synth.indptr(w.kv_lens) + start
    return RaggedCase(w, q, rows[0], rows[1], kv_ind, synth.indptr(w.qo_lens))


def make_ragged_plan(case: RaggedCase, num_cus: int = 0,
                     kv_chunk_tokens: Optional[int] = None, rope: Optional[tuple] = None) -> Plan:
    w = case.w
    chunk = w.kv_chunk_tokens if kv_chunk_tokens is None else kv_chunk_tokens
    theta, scale = rope if rope is not None else (None, 1.0)
    return Plan(w.kv_lens, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                head_dim_qk=w.head_dim_qk, head_dim_vo=w.head_dim_vo,
                qo_indptr=case.qo_indptr.tolist(), kv_indptr=case.kv_indptr.tolist(),
                causal=w.causal, kv_chunk_tokens=chunk, num_cus=num_cus, kv_dtype=case.k.dtype,
                rope_theta=theta, rope_scale=scale)
