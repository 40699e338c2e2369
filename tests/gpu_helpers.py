"""Test-side construction of paged NVFP4 caches whose bytes come from the oracle's
own quantiser, plus the comparison rules used by the GPU parity tests.

Tolerances: O max |error| <= 1e-2, LSE |error| <= 1e-3 * max(1, |LSE|), and the
least-squares scale alpha = <o, ref> / <ref, ref> within [0.99, 1.01] (a uniform
scale error that a loose absolute bound could absorb fails this)."""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import synth
from oracle import nvfp4_ref as ref

O_ATOL = 1e-2
LSE_RTOL = 1e-3


@dataclasses.dataclass
class OracleCase:
    w: synth.Workload
    layout: str
    q_np: np.ndarray
    k_np: tuple   # (data, sf) numpy views the oracle reads
    v_np: tuple
    pt: np.ndarray
    q: torch.Tensor
    k_pool: nv.KVPool
    v_pool: nv.KVPool
    page_table: torch.Tensor
    k_global: float
    v_global: float
    kv_dtype: str = "nvfp4"


def _pool_arrays(w, layout, packed, sf, slots, head_dim, pad, seed):
    """numpy pool (data, sf) with random bytes / NaN scales everywhere, rows at their slots.
    ``pad`` = (pages, heads, tokens, bytes) of extra parent padding -> unequal strides.
    ``sf`` None: an FP8 pool (rows of head_dim bytes, no scale pool)."""
    P, H = w.page_size, w.num_kv_heads
    rng = np.random.default_rng(seed)
    pp, ph, pt_, pb = pad
    row = head_dim // 2 if sf is not None else head_dim
    if layout == "HND":
        dshape = (w.pool_pages + pp, H + ph, P + pt_, row + pb)
        sshape = (w.pool_pages + pp, H + ph, P + pt_, head_dim // 16 + (8 if pb else 0))
    else:
        dshape = (w.pool_pages + pp, P + pt_, H + ph, row + pb)
        sshape = (w.pool_pages + pp, P + pt_, H + ph, head_dim // 16 + (8 if pb else 0))
    dpar = rng.integers(0, 256, dshape, dtype=np.uint8)
    spar = np.full(sshape, synth.SF_POISON, dtype=np.uint8) if sf is not None else None
    lead = (slice(0, w.pool_pages), slice(0, H), slice(0, P)) if layout == "HND" else \
        (slice(0, w.pool_pages), slice(0, P), slice(0, H))
    d = dpar[lead + (slice(0, row),)]
    s = spar[lead + (slice(0, head_dim // 16),)] if sf is not None else None
    pages, offs = slots // P, slots % P
    if layout == "HND":
        d[pages, :, offs, :] = packed
        if s is not None:
            s[pages, :, offs, :] = sf
    else:
        d[pages, offs, :, :] = packed
        if s is not None:
            s[pages, offs, :, :] = sf
    return dpar, spar, d, s


def _to_device_view(parent, view, device):
    t = torch.from_numpy(np.ascontiguousarray(parent)).to(device)
    idx = tuple(slice(0, n) for n in view.shape)
    return t[idx]


def build_oracle_case(w: synth.Workload, layout="HND", device="cuda", k_global=1.0,
                      v_global=1.0, k_pad=(0, 0, 0, 0), v_pad=(0, 0, 0, 0),
                      pad_page: Optional[int] = None, kv_dtype: str = "nvfp4") -> OracleCase:
    q, k, v = synth.draw_qkv(w, device="cpu")
    if kv_dtype == "fp8":
        kq, ks = ref.quantize_fp8(k.double().numpy(), k_global), None
        vq, vs = ref.quantize_fp8(v.double().numpy(), v_global), None
    else:
        kq, ks = ref.quantize(k.double().numpy(), k_global)
        vq, vs = ref.quantize(v.double().numpy(), v_global)
    pt = synth.page_table(w, pad_page)
    slots = synth.token_slots(w, pt)
    kd_par, ks_par, kd, ksf = _pool_arrays(w, layout, kq, ks, slots, w.head_dim_qk, k_pad, 1)
    vd_par, vs_par, vd, vsf = _pool_arrays(w, layout, vq, vs, slots, w.head_dim_vo, v_pad, 2)
    dv = lambda par, view: None if par is None else _to_device_view(par, view, device)
    k_pool = nv.KVPool(dv(kd_par, kd), dv(ks_par, ksf), head_dim=w.head_dim_qk, layout=layout,
                       global_scale=k_global, dtype=kv_dtype)
    v_pool = nv.KVPool(dv(vd_par, vd), dv(vs_par, vsf), head_dim=w.head_dim_vo, layout=layout,
                       global_scale=v_global, dtype=kv_dtype)
    return OracleCase(w, layout, q.double().numpy(), (kd, ksf), (vd, vsf), pt, q.to(device),
                      k_pool, v_pool, torch.from_numpy(pt).to(device), k_global, v_global,
                      kv_dtype)


def oracle_reference(c: OracleCase, rows=None):
    w = c.w
    return ref.paged_attention(c.q_np, c.k_np[0], c.k_np[1], c.v_np[0], c.v_np[1], c.pt,
                               w.kv_lens, synth.indptr(w.qo_lens), w.page_size, w.sm_scale,
                               w.causal, c.layout, c.k_global, c.v_global, rows=rows,
                               kv_dtype=c.kv_dtype)


def make_plan(w: synth.Workload, chunk=None, num_cus=256, kv_dtype="nvfp4"):
    return nv.Plan(w.kv_lens, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                   head_dim_qk=w.head_dim_qk, head_dim_vo=w.head_dim_vo, page_size=w.page_size,
                   qo_indptr=None if w.decode else synth.indptr(w.qo_lens).tolist(),
                   causal=w.causal, kv_chunk_tokens=w.kv_chunk_tokens if chunk is None else chunk,
                   num_cus=num_cus, kv_dtype=kv_dtype)


def run_gpu(c: OracleCase, plan: nv.Plan):
    ws = plan.new_workspace(c.q.device)
    plan.upload(ws)
    rows = c.q.shape[0]
    o = torch.full((rows, c.w.num_qo_heads, c.w.head_dim_vo), float("nan"), device=c.q.device)
    lse = torch.full((rows, c.w.num_qo_heads), float("nan"), device=c.q.device)
    fn = nv.batch_decode if c.w.decode else nv.batch_prefill
    fn(plan, c.q, c.page_table, c.k_pool, c.v_pool, c.w.sm_scale, ws, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def assert_attention_close(o, lse, o_ref, lse_ref, what=""):
    sel = ~np.isnan(lse_ref)
    assert sel.any()
    o, lse, o_ref, lse_ref = o[sel], lse[sel], o_ref[sel], lse_ref[sel]
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    err = np.abs(o - o_ref).max() if o.size else 0.0
    assert err <= O_ATOL, f"{what}: max |O err| = {err:.3e}"
    inf = np.isinf(lse_ref)
    assert np.array_equal(np.isinf(lse), inf), f"{what}: -inf LSE rows differ"
    if (~inf).any():
        lerr = (np.abs(lse[~inf] - lse_ref[~inf]) / np.maximum(1.0, np.abs(lse_ref[~inf]))).max()
        assert lerr <= LSE_RTOL, f"{what}: max relative LSE err = {lerr:.3e}"
    den = float((o_ref * o_ref).sum())
    if den > 0:
        alpha = float((o * o_ref).sum()) / den
        assert 0.99 <= alpha <= 1.01, f"{what}: alpha = {alpha}"
    return err
