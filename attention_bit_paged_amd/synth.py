"""Seeded synthetic inputs for NVFP4 paged attention.

This module only draws random numbers and lays out page tables. It holds none
of the attention or quantisation arithmetic, so that the CPU reference and the
HIP path can both consume exactly the same inputs without sharing any of the
method's code.

Recipe (the same for every workload):
  * values: Q, then K, then V are drawn in that order from one torch generator
    seeded with ``value_seed`` as float32 N(0, 1) and rounded to bfloat16 (RNE);
    K and V are drawn for the concatenation of all requests' tokens;
  * lengths: ``numpy.random.default_rng(length_seed).integers(lo, hi,
    endpoint=True)``;
  * pages: a ``default_rng(page_seed).permutation(pool_pages)``; request b takes
    the next ceil(L_b / page_size) pages in order;
  * sm_scale = 1 / sqrt(head_dim_qk).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention workload over a paged NVFP4 KV cache."""

    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_vo: int
    page_size: int
    kv_lens: tuple            # total kv length per request (prefix + new)
    qo_lens: tuple            # query rows per request (1 for decode)
    causal: bool
    pool_pages: int           # pages in the K (and V) pool
    permute_pages: bool
    value_seed: int
    page_seed: int
    kv_chunk_tokens: int      # 0 = let the planner choose
    decode: bool

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim_qk)

    @property
    def total_q(self) -> int:
        return int(sum(self.qo_lens))

    @property
    def total_kv(self) -> int:
        return int(sum(self.kv_lens))

    def pages_needed(self) -> int:
        return int(sum(-(-l // self.page_size) for l in self.kv_lens))

    def kv_bytes(self, dtype: str = "nvfp4") -> int:
        """Bytes of every visible K and V row: packed e2m1 bytes plus e4m3 scale bytes
        (NVFP4), or one byte per element (FP8)."""
        if dtype == "fp8":
            per_tok = self.head_dim_qk + self.head_dim_vo
        else:
            per_tok = (self.head_dim_qk // 2 + self.head_dim_qk // 16
                       + self.head_dim_vo // 2 + self.head_dim_vo // 16)
        return self.total_kv * self.num_kv_heads * per_tok

    def unmasked_pairs(self) -> int:
        """Number of (query row, key) pairs that the mask leaves visible, per qo head."""
        n = 0
        for q, l in zip(self.qo_lens, self.kv_lens):
            if self.causal:
                prefix = l - q
                n += q * prefix + q * (q + 1) // 2
            else:
                n += q * l
        return n

    def flops(self) -> int:
        """2 * (Dk + Dv) multiply-adds per visible (query, key) pair and qo head."""
        return 2 * (self.head_dim_qk + self.head_dim_vo) * self.num_qo_heads * self.unmasked_pairs()


def _lengths(seed: int, lo: int, hi: int, n: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(lo, hi, size=n, endpoint=True)


def workload(name: str, **overrides) -> Workload:
    """The named workloads.  Seeds: values 1000+i, lengths 2000+i, pages 3000+i."""
    if name == "single_decode":           # B1, L128, 4/1 heads, D128, contiguous
        w = dict(batch=1, num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, head_dim_vo=128,
                 kv_lens=(128,), qo_lens=(1,), causal=False, pool_pages=8, permute_pages=False,
                 idx=1, kv_chunk_tokens=0, decode=True)
    elif name == "batch_decode":          # B64, L~U[512,8192], 32/8, D128, 40k pool
        lens = _lengths(2002, 512, 8192, 64)
        w = dict(batch=64, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_vo=128,
                 kv_lens=tuple(int(x) for x in lens), qo_lens=(1,) * 64, causal=False,
                 pool_pages=40000, permute_pages=True, idx=2, kv_chunk_tokens=256, decode=True)
    elif name == "long_decode":           # B8, L131072, 32/8, D128
        w = dict(batch=8, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_vo=128,
                 kv_lens=(131072,) * 8, qo_lens=(1,) * 8, causal=False, pool_pages=65536,
                 permute_pages=True, idx=3, kv_chunk_tokens=0, decode=True)
    elif name == "prefill_extend":        # B16, prefix~U[0,4096], q~U[128,512], causal
        rng_pref = _lengths(2004, 0, 4096, 16)
        rng_q = np.random.default_rng(2104).integers(128, 512, size=16, endpoint=True)
        kv = tuple(int(p + q) for p, q in zip(rng_pref, rng_q))
        pool = sum(-(-l // 16) for l in kv)
        w = dict(batch=16, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_vo=128,
                 kv_lens=kv, qo_lens=tuple(int(q) for q in rng_q), causal=True,
                 pool_pages=pool + 64, permute_pages=True, idx=4, kv_chunk_tokens=0, decode=False)
    elif name == "asym_prefill":          # B4, q = L = 1024 causal, 8/1, 512/256
        w = dict(batch=4, num_qo_heads=8, num_kv_heads=1, head_dim_qk=512, head_dim_vo=256,
                 kv_lens=(1024,) * 4, qo_lens=(1024,) * 4, causal=True, pool_pages=4 * 64 + 16,
                 permute_pages=True, idx=5, kv_chunk_tokens=0, decode=False)
    elif name == "asym_decode":           # B32, L32768, 8/1, 512/256
        w = dict(batch=32, num_qo_heads=8, num_kv_heads=1, head_dim_qk=512, head_dim_vo=256,
                 kv_lens=(32768,) * 32, qo_lens=(1,) * 32, causal=False, pool_pages=32 * 2048 + 64,
                 permute_pages=True, idx=6, kv_chunk_tokens=0, decode=True)
    else:
        raise ValueError(f"unknown workload {name!r}")
    idx = w.pop("idx")
    w.update(name=name, page_size=16, value_seed=1000 + idx, page_seed=3000 + idx)
    w.update(overrides)
    return Workload(**w)


WORKLOADS = ("single_decode", "batch_decode", "long_decode", "prefill_extend",
             "asym_prefill", "asym_decode")


def custom(name="custom", *, kv_lens: Sequence[int], qo_lens: Optional[Sequence[int]] = None,
           num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, head_dim_vo=None, page_size=16,
           causal=False, extra_pages=3, permute_pages=True, seed=7,
           kv_chunk_tokens=0) -> Workload:
    """A small workload for tests."""
    head_dim_vo = head_dim_qk if head_dim_vo is None else head_dim_vo
    decode = qo_lens is None
    qo_lens = tuple([1] * len(kv_lens)) if decode else tuple(int(x) for x in qo_lens)
    kv_lens = tuple(int(x) for x in kv_lens)
    pages = sum(-(-l // page_size) for l in kv_lens) + extra_pages
    return Workload(name=name, batch=len(kv_lens), num_qo_heads=num_qo_heads,
                    num_kv_heads=num_kv_heads, head_dim_qk=head_dim_qk, head_dim_vo=head_dim_vo,
                    page_size=page_size, kv_lens=kv_lens, qo_lens=qo_lens, causal=causal,
                    pool_pages=max(pages, 1), permute_pages=permute_pages, value_seed=seed,
                    page_seed=seed + 1, kv_chunk_tokens=kv_chunk_tokens, decode=decode)


def draw_qkv(w: Workload, device="cpu"):
    """Q [sum q, Hq, Dk], K [sum L, Hkv, Dk], V [sum L, Hkv, Dv] in bfloat16, drawn in that order."""
    g = torch.Generator(device=device)
    g.manual_seed(w.value_seed)
    out = []
    for shape in ((w.total_q, w.num_qo_heads, w.head_dim_qk),
                  (w.total_kv, w.num_kv_heads, w.head_dim_qk),
                  (w.total_kv, w.num_kv_heads, w.head_dim_vo)):
        out.append(torch.randn(shape, generator=g, dtype=torch.float32, device=device)
                   .to(torch.bfloat16))
    return tuple(out)


def page_assignment(w: Workload) -> np.ndarray:
    """Physical page order: a seeded permutation of the pool (or 0..n-1)."""
    if w.permute_pages:
        return np.random.default_rng(w.page_seed).permutation(w.pool_pages).astype(np.int32)
    return np.arange(w.pool_pages, dtype=np.int32)


def page_table(w: Workload, pad_page: Optional[int] = None) -> np.ndarray:
    """int32 [batch, max_pages]; request b takes the next ceil(L_b/P) pages of the assignment.

    Entries past a request's last page are set to ``pad_page`` (default: the
    last page of the assignment, which no request uses when the pool has spare
    pages), so a stray read lands on a poisoned page rather than out of bounds.
    """
    order = page_assignment(w)
    counts = [-(-l // w.page_size) for l in w.kv_lens]
    need = sum(counts)
    if need > w.pool_pages:
        raise ValueError(f"pool of {w.pool_pages} pages cannot hold {need}")
    max_pages = max(max(counts), 1)
    pad = int(order[-1]) if pad_page is None else int(pad_page)
    pt = np.full((w.batch, max_pages), pad, dtype=np.int32)
    pos = 0
    for b, c in enumerate(counts):
        pt[b, :c] = order[pos:pos + c]
        pos += c
    return pt


def token_slots(w: Workload, pt: np.ndarray) -> np.ndarray:
    """int64 slot (page * page_size + offset) of every K/V token, requests concatenated."""
    slots = np.empty(w.total_kv, dtype=np.int64)
    pos = 0
    for b, l in enumerate(w.kv_lens):
        j = np.arange(l)
        slots[pos:pos + l] = pt[b, j // w.page_size].astype(np.int64) * w.page_size + j % w.page_size
        pos += l
    return slots


def indptr(lens: Sequence[int]) -> np.ndarray:
    out = np.zeros(len(lens) + 1, dtype=np.int32)
    out[1:] = np.cumsum(lens)
    return out


def poison_bytes(shape, seed: int) -> np.ndarray:
    """Random packed bytes for pool slots that no request should read."""
    return np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)


# e4m3fn byte 0x7F is NaN: a scale slot filled with it poisons any stray read.
SF_POISON = 0x7F
