"""NVFP4 paged-KV attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/nvfp4_attn.h``.  PyTorch supplies
device memory and the current stream; every step of the computation runs in the
HIP library (``libnvfp4_attn.so``).  The names follow the C entry points:
``quantize_kv``, ``Plan`` (``nvfp4_plan_*``), ``batch_decode``, ``batch_prefill``
and ``merge_states``.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from ._lib import (EXPORTS, KV_DTYPES, STATUS, WORK_FIELDS, KVPoolStruct, KVRaggedStruct,
                   POS_ENCODINGS, NVFP4Error, PlanInfoStruct, PlanOptionsStruct, check, lib)

__all__ = ["KVPool", "RaggedKV", "Plan", "Prepared", "quantize_kv", "batch_decode",
           "batch_decode_noalloc", "batch_decode_append", "batch_prefill", "batch_prefill_masked",
           "batch_prefill_ragged", "kv_checksum",
           "merge_partials", "merge_states", "NVFP4Error", "lib", "version", "EXPORTS"]


def version() -> str:
    return lib.nvfp4_version().decode()


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _device(*tensors) -> torch.device:
    """The one GPU every given tensor lives on (None entries are skipped).  The kernels
    dereference these pointers on the device: a host tensor, or one on another GPU,
    would fault there, so it is refused here, before any library call."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor passed to the library must be a GPU tensor "
                             f"(got one on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")
    if dev is None:
        raise ValueError("no GPU tensor given")
    return dev


def _stream(stream, device: Optional[torch.device] = None) -> ctypes.c_void_p:
    """The stream to launch on: by default the current stream of ``device``; a given
    stream must belong to ``device``."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif device is not None and stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
    return ctypes.c_void_p(stream.cuda_stream)


def _row_bytes(head_dim: int, dtype: str) -> int:
    return head_dim if dtype == "fp8" else head_dim // 2


class KVPool:
    """One paged pool (K or V) of NVFP4 (``dtype="nvfp4"``) or FP8 e4m3 (``"fp8"``).

    ``data`` is uint8 ``[pages, H, P, W]`` (layout "HND") or ``[pages, P, H, W]``
    ("NHD") with W = D/2 (NVFP4) or D (FP8); an NVFP4 pool's ``sf`` has the same leading
    dims and ``D/16`` scale bytes, an FP8 pool has none (``sf=None``).  Any strides are
    allowed as long as the last dimension is contiguous.
    """

    def __init__(self, data: torch.Tensor, sf: Optional[torch.Tensor], *, head_dim: int,
                 layout="HND", global_scale: float = 1.0, dtype: str = "nvfp4"):
        if dtype not in KV_DTYPES:
            raise ValueError(f"dtype must be one of {sorted(KV_DTYPES)}, got {dtype!r}")
        if (sf is None) != (dtype == "fp8"):
            raise ValueError("an NVFP4 pool needs its scale tensor; an FP8 pool has none")
        if data.dtype != torch.uint8 or (sf is not None and sf.dtype != torch.uint8):
            raise TypeError("pool data and scales must be uint8 tensors")
        if data.dim() != 4 or (sf is not None and sf.dim() != 4):
            raise ValueError("pool tensors must be 4-D")
        if layout not in ("HND", "NHD"):
            raise ValueError(f"layout must be HND or NHD, got {layout!r}")
        if data.stride(-1) != 1 or (sf is not None and sf.stride(-1) != 1):
            raise ValueError("the last pool dimension must be contiguous")
        if sf is not None and tuple(data.shape[:3]) != tuple(sf.shape[:3]):
            raise ValueError("pool data and scales must have the same leading dims")
        if sf is not None and data.device != sf.device:
            raise ValueError("pool data and scales must be on one device")
        self.data, self.sf, self.layout, self.dtype = data, sf, layout, dtype
        self.head_dim = int(head_dim)
        self.global_scale = float(global_scale)
        self.num_pages = data.shape[0]
        if layout == "HND":
            self.num_kv_heads, self.page_size = data.shape[1], data.shape[2]
        else:
            self.page_size, self.num_kv_heads = data.shape[1], data.shape[2]
        if data.shape[-1] != _row_bytes(head_dim, dtype) or \
                (sf is not None and sf.shape[-1] != head_dim // 16):
            raise ValueError("pool last dims must be head_dim/2 (NVFP4 data) or head_dim (FP8 "
                             "data), and head_dim/16 (scales)")

    def tensors(self):
        return (self.data,) if self.sf is None else (self.data, self.sf)

    @classmethod
    def empty(cls, num_pages: int, num_kv_heads: int, page_size: int, head_dim: int,
              layout="HND", device="cuda", global_scale: float = 1.0,
              dtype: str = "nvfp4") -> "KVPool":
        if layout == "HND":
            shape = (num_pages, num_kv_heads, page_size)
        else:
            shape = (num_pages, page_size, num_kv_heads)
        data = torch.empty(shape + (_row_bytes(head_dim, dtype),), dtype=torch.uint8,
                           device=device)
        sf = None if dtype == "fp8" else torch.empty(shape + (head_dim // 16,), dtype=torch.uint8,
                                                     device=device)
        return cls(data, sf, head_dim=head_dim, layout=layout, global_scale=global_scale,
                   dtype=dtype)

    def struct(self) -> KVPoolStruct:
        """The C view of this pool (built once: the tensors of a pool never change)."""
        if getattr(self, "_struct", None) is None:
            self._struct = self._make_struct()
        return self._struct

    def _make_struct(self) -> KVPoolStruct:
        d = self.data.stride()
        s = self.sf.stride() if self.sf is not None else (0, 0, 0, 1)
        if self.layout == "HND":
            dp, dh, dt = d[0], d[1], d[2]
            sp, sh, st = s[0], s[1], s[2]
        else:
            dp, dt, dh = d[0], d[1], d[2]
            sp, st, sh = s[0], s[1], s[2]
        return KVPoolStruct(self.data.data_ptr(), dp, dh, dt,
                            self.sf.data_ptr() if self.sf is not None else None, sp, sh, st,
                            self.num_pages, self.page_size, self.num_kv_heads, self.head_dim,
                            self.global_scale, KV_DTYPES[self.dtype])


class RaggedKV:
    """Ragged (non-paged) K or V rows for ``batch_prefill_ragged``: ``data`` uint8
    ``[rows, H, W]`` (W = D/2 for NVFP4, D for FP8) and, for NVFP4, ``sf`` ``[rows, H,
    D/16]``.  Request b's keys are rows ``kv_indptr[b] .. kv_indptr[b+1]-1``; rows are
    streamed in 16-row pages, so up to 15 rows past the last request must exist
    (``empty`` adds them)."""

    def __init__(self, data: torch.Tensor, sf: Optional[torch.Tensor], *, head_dim: int,
                 global_scale: float = 1.0, dtype: str = "nvfp4"):
        if dtype not in KV_DTYPES:
            raise ValueError(f"dtype must be one of {sorted(KV_DTYPES)}, got {dtype!r}")
        if (sf is None) != (dtype == "fp8"):
            raise ValueError("NVFP4 rows need their scale tensor; FP8 rows have none")
        for t in (data, sf):
            if t is not None and (t.dtype != torch.uint8 or t.dim() != 3 or t.stride(-1) != 1):
                raise ValueError("ragged tensors must be uint8 [rows, heads, bytes] with a "
                                 "contiguous last dim")
        if data.shape[-1] != _row_bytes(head_dim, dtype) or \
                (sf is not None and (sf.shape[-1] != head_dim // 16 or sf.shape[:2] != data.shape[:2])):
            raise ValueError("ragged rows must hold head_dim/2 (NVFP4) or head_dim (FP8) bytes "
                             "and head_dim/16 scale bytes")
        self.data, self.sf, self.dtype = data, sf, dtype
        self.head_dim, self.global_scale = int(head_dim), float(global_scale)
        self.num_rows, self.num_kv_heads = data.shape[0], data.shape[1]

    @classmethod
    def empty(cls, total_rows: int, num_kv_heads: int, head_dim: int, device="cuda",
              global_scale: float = 1.0, dtype: str = "nvfp4") -> "RaggedKV":
        rows = total_rows + 15
        data = torch.empty((rows, num_kv_heads, _row_bytes(head_dim, dtype)), dtype=torch.uint8,
                           device=device)
        sf = None if dtype == "fp8" else torch.empty((rows, num_kv_heads, head_dim // 16),
                                                     dtype=torch.uint8, device=device)
        return cls(data, sf, head_dim=head_dim, global_scale=global_scale, dtype=dtype)

    def tensors(self):
        return (self.data,) if self.sf is None else (self.data, self.sf)

    def struct(self) -> KVRaggedStruct:
        s = self.sf.stride() if self.sf is not None else (0, 0, 1)
        return KVRaggedStruct(self.data.data_ptr(), self.data.stride(0), self.data.stride(1),
                              self.sf.data_ptr() if self.sf is not None else None, s[0], s[1],
                              self.num_rows, self.num_kv_heads, self.head_dim, self.global_scale,
                              KV_DTYPES[self.dtype])


class Prepared:
    """One library call with its arguments marshalled once (``prepare=True`` on the
    calls below).  Calling it launches again on the same stream with the same tensors,
    whose contents may change between calls but whose storage must stay alive; it
    keeps references to them.  For launch loops where per-call Python work matters."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self) -> None:
        check(self._fn(*self._args))


def quantize_kv(k: Optional[torch.Tensor], v: Optional[torch.Tensor], slot_mapping: torch.Tensor,
                k_pool: Optional[KVPool], v_pool: Optional[KVPool], stream=None,
                prepare: bool = False):
    """Quantise bf16 K/V rows ``[n_tokens, H, D]`` into their pools at ``slot_mapping``
    (int64 ``page * page_size + offset``; negative = skip)."""
    if (k is None) != (k_pool is None) or (v is None) != (v_pool is None):
        raise ValueError("each source needs its pool and each pool its source")
    if k is None and v is None:
        raise ValueError("nothing to quantise")
    n = (k if k is not None else v).shape[0]
    for name, t, pool in (("k", k, k_pool), ("v", v, v_pool)):
        if t is None:
            continue
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be bf16 [n_tokens, heads, head_dim], last dim contiguous")
        # the kernel reads n_tokens x heads x head_dim elements of each source
        if tuple(t.shape) != (n, pool.num_kv_heads, pool.head_dim):
            raise ValueError(f"{name} must have shape ({n}, {pool.num_kv_heads}, {pool.head_dim}) "
                             f"to match its pool, got {tuple(t.shape)}")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1 \
            or slot_mapping.numel() != n or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 vector with one entry per token")
    dev = _device(k, v, slot_mapping, *(t for p in (k_pool, v_pool) if p is not None
                                        for t in p.tensors()))
    ks = k_pool.struct() if k_pool is not None else None
    vs = v_pool.struct() if v_pool is not None else None
    args = (_ptr(k), k.stride(0) if k is not None else 0, k.stride(1) if k is not None else 0,
            _ptr(v), v.stride(0) if v is not None else 0, v.stride(1) if v is not None else 0,
            n, _ptr(slot_mapping),
            ctypes.byref(ks) if ks is not None else None,
            ctypes.byref(vs) if vs is not None else None, _stream(stream, dev))
    if prepare:
        return Prepared(lib.nvfp4_quantize_kv, args, (k, v, slot_mapping, k_pool, v_pool, ks, vs))
    check(lib.nvfp4_quantize_kv(*args))


class Plan:
    """Host-side split of one batch into work items (``nvfp4_plan_create``).

    Decode when ``qo_indptr`` is None (one query per request), else prefill.
    """

    def __init__(self, kv_lens: Sequence[int], *, num_qo_heads: int, num_kv_heads: int,
                 head_dim_qk: int, head_dim_vo: Optional[int] = None, page_size: int = 16,
                 qo_indptr: Optional[Sequence[int]] = None, causal: bool = False,
                 kv_chunk_tokens: int = 0, num_cus: int = 0, device=None,
                 kv_dtype: str = "nvfp4", kv_indptr: Optional[Sequence[int]] = None,
                 custom_mask: bool = False, rope_theta: Optional[float] = None,
                 rope_scale: float = 1.0):
        """``num_cus`` 0 fills the compute units of ``device`` (default: the current
        device when a GPU is present, else the library's default of 256).  ``kv_dtype``:
        the pools' type ("nvfp4" or "fp8"); ``kv_indptr``: ragged (non-paged) prefill KV
        rows per request; ``custom_mask``: runs take a packed mask in place of the causal
        rule; ``rope_theta``: the prefill kernels apply the rotary embedding (base
        ``rope_theta``, positions divided by ``rope_scale``) to Q and K
        (nvfp4_plan_create_ex)."""
        head_dim_vo = head_dim_qk if head_dim_vo is None else head_dim_vo
        if kv_dtype not in KV_DTYPES:
            raise ValueError(f"kv_dtype must be one of {sorted(KV_DTYPES)}, got {kv_dtype!r}")
        self.kv_dtype = kv_dtype
        self._kvind = None if kv_indptr is None else np.ascontiguousarray(
            np.asarray(kv_indptr, dtype=np.int32))
        self.ragged = kv_indptr is not None
        self.custom_mask = bool(custom_mask)
        self.rope = None if rope_theta is None else (float(rope_theta), float(rope_scale))
        if num_cus == 0 and torch.cuda.is_available():
            num_cus = torch.cuda.get_device_properties(
                torch.device("cuda") if device is None else torch.device(device)
            ).multi_processor_count
        self._kv = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
        self._ind = None if qo_indptr is None else np.ascontiguousarray(
            np.asarray(qo_indptr, dtype=np.int32))
        self._h = ctypes.c_void_p()
        # held on the instance: module globals may already be gone when a plan is
        # collected at interpreter exit
        self._destroy = lib.nvfp4_plan_destroy
        self.batch = len(self._kv)
        self.num_qo_heads, self.num_kv_heads = num_qo_heads, num_kv_heads
        self.head_dim_qk, self.head_dim_vo, self.page_size = head_dim_qk, head_dim_vo, page_size
        self.causal = causal
        opts = PlanOptionsStruct(KV_DTYPES[kv_dtype], None if self._kvind is None
                                 else self._kvind.ctypes.data_as(ctypes.c_void_p).value,
                                 int(self.custom_mask),
                                 POS_ENCODINGS["none" if self.rope is None else "rope"],
                                 *(self.rope or (0.0, 0.0)))
        check(lib.nvfp4_plan_create_ex(
            self._kv.ctypes.data_as(ctypes.c_void_p) if self.batch else None,
            self._ind.ctypes.data_as(ctypes.c_void_p) if self._ind is not None else None,
            self.batch, num_qo_heads, num_kv_heads, head_dim_qk, head_dim_vo, page_size,
            int(bool(causal)), kv_chunk_tokens, num_cus, ctypes.byref(opts),
            ctypes.byref(self._h)))
        if self.ragged:
            self.page_size = 16

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    @property
    def workspace_bytes(self) -> int:
        return int(lib.nvfp4_plan_workspace_bytes(self._h))

    def info(self) -> dict:
        s = PlanInfoStruct()
        check(lib.nvfp4_plan_get_info(self._h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in PlanInfoStruct._fields_}

    def work(self) -> np.ndarray:
        n = self.info()["num_work_items"]
        out = np.zeros((max(n, 1), len(WORK_FIELDS)), dtype=np.int32)
        check(lib.nvfp4_plan_get_work(self._h, out.ctypes.data_as(ctypes.c_void_p), n))
        return out[:n]

    def new_workspace(self, device="cuda") -> torch.Tensor:
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device)

    def upload(self, workspace: torch.Tensor, stream=None) -> None:
        _check_workspace(self, workspace)
        check(lib.nvfp4_plan_upload(self._h, _ptr(workspace), workspace.numel(),
                                    _stream(stream, _device(workspace))))

    @property
    def mask_bytes(self) -> int:
        """Bytes of the packed custom mask of this plan's requests (without the 8 bytes
        of read-ahead the buffer must also hold)."""
        return int(lib.nvfp4_plan_mask_bytes(self._h))

    @property
    def total_rows(self) -> int:
        """Query rows of the batch: one per request (decode) or qo_indptr[-1]."""
        return self.batch if self._ind is None else int(self._ind[-1])

    def max_pages(self) -> int:
        """Page-table columns the longest request needs."""
        if self.batch == 0:
            return 0
        return int(max(-(-int(l) // self.page_size) for l in self._kv))

    def set_deferred_merge(self, deferred: bool = True) -> None:
        """Runs leave split rows' partials for ``merge_partials`` (nvfp4_plan_set_deferred_merge)."""
        check(lib.nvfp4_plan_set_deferred_merge(self._h, int(bool(deferred))))


def _check_workspace(plan: Plan, ws: torch.Tensor):
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous() \
            or ws.numel() < plan.workspace_bytes:
        raise ValueError(f"workspace must be a contiguous uint8 vector of at least "
                         f"{plan.workspace_bytes} bytes")


def _check_outputs(plan: Plan, out, lse):
    """out fp32 [rows, Hq, Dv] with a contiguous last dim, lse fp32 [rows, Hq] contiguous."""
    rows = plan.total_rows
    for name, t, shape in (("out", out, (rows, plan.num_qo_heads, plan.head_dim_vo)),
                           ("lse", lse, (rows, plan.num_qo_heads))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    if out is not None and (out.dtype != torch.float32 or out.stride(-1) != 1):
        raise ValueError("out must be fp32 with a contiguous last dim")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be fp32 and contiguous")


def _check_rows(plan: Plan, q, page_table, out, lse):
    """Shapes the C library cannot see (it takes pointers): q, page table and outputs
    must cover the plan's rows, or the kernels would read or write past them."""
    rows = plan.total_rows
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.stride(-1) != 1 \
            or tuple(q.shape) != (rows, plan.num_qo_heads, plan.head_dim_qk):
        raise ValueError(f"q must be bf16 [{rows}, {plan.num_qo_heads}, {plan.head_dim_qk}] "
                         "with a contiguous last dim")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.stride(1) != 1 \
            or page_table.shape[0] < plan.batch or page_table.shape[1] < plan.max_pages():
        raise ValueError(f"page_table must be int32 [>= {plan.batch}, >= {plan.max_pages()}] "
                         "with contiguous rows")
    _check_outputs(plan, out, lse)
    return rows


def _check_pools(plan: Plan, k_pool: "KVPool", v_pool: "KVPool"):
    if plan.ragged:
        raise ValueError("the plan was made for ragged KV rows: use batch_prefill_ragged")
    for name, p, d in (("k_pool", k_pool, plan.head_dim_qk), ("v_pool", v_pool, plan.head_dim_vo)):
        if p.head_dim != d or p.num_kv_heads != plan.num_kv_heads or p.page_size != plan.page_size:
            raise ValueError(f"{name} is (heads {p.num_kv_heads}, page {p.page_size}, dim "
                             f"{p.head_dim}); the plan needs ({plan.num_kv_heads}, "
                             f"{plan.page_size}, {d})")
        if p.dtype != plan.kv_dtype:
            raise ValueError(f"{name} holds {p.dtype}, the plan was made for {plan.kv_dtype}")


def _attn(fn, plan: Plan, q, page_table, k_pool, v_pool, sm_scale, workspace, out, lse, stream,
          prepare=False):
    if plan.custom_mask:
        raise ValueError("the plan was made for a custom mask: use batch_prefill_masked")
    rows = _check_rows(plan, q, page_table, out, lse)
    _check_pools(plan, k_pool, v_pool)
    _check_workspace(plan, workspace)
    dev = _device(q, page_table, *k_pool.tensors(), *v_pool.tensors(), workspace, out, lse)
    if out is None:
        out = torch.empty((rows, plan.num_qo_heads, plan.head_dim_vo), dtype=torch.float32,
                          device=dev)
    if lse is None:
        lse = torch.empty((rows, plan.num_qo_heads), dtype=torch.float32, device=dev)
    ks, vs = k_pool.struct(), v_pool.struct()
    args = (plan.handle, _ptr(q), q.stride(0), q.stride(1), _ptr(page_table), page_table.stride(0),
            ctypes.byref(ks), ctypes.byref(vs), float(sm_scale), _ptr(workspace),
            workspace.numel(), _ptr(out), out.stride(0), out.stride(1), _ptr(lse),
            _stream(stream, dev))
    if prepare:
        return Prepared(fn, args, (plan, q, page_table, k_pool, v_pool, ks, vs, workspace, out, lse))
    check(fn(*args))
    return out, lse


def batch_decode(plan: Plan, q: torch.Tensor, page_table: torch.Tensor, k_pool: KVPool,
                 v_pool: KVPool, sm_scale: float, workspace: torch.Tensor,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 stream=None, prepare: bool = False):
    """Decode attention; returns (O fp32 [batch, Hq, Dv], LSE fp32 [batch, Hq]), or a
    ``Prepared`` call with ``prepare=True``."""
    return _attn(lib.nvfp4_batch_decode, plan, q, page_table, k_pool, v_pool, sm_scale,
                 workspace, out, lse, stream, prepare)


def batch_decode_noalloc(plan: Plan, q: torch.Tensor, page_table: torch.Tensor, k_pool: KVPool,
                         v_pool: KVPool, sm_scale: float, out: torch.Tensor, lse: torch.Tensor,
                         stream=None):
    """Decode with the library's fixed per-GPU scratch in place of a workspace
    (nvfp4_batch_decode_noalloc): allocates nothing, so ``out`` and ``lse`` must be
    given.  Calls that overlap on one GPU race on the shared scratch."""
    if out is None or lse is None:
        raise ValueError("out and lse must be given: the call allocates nothing")
    _check_rows(plan, q, page_table, out, lse)
    _check_pools(plan, k_pool, v_pool)
    dev = _device(q, page_table, *k_pool.tensors(), *v_pool.tensors(), out, lse)
    ks, vs = k_pool.struct(), v_pool.struct()
    check(lib.nvfp4_batch_decode_noalloc(
        plan.handle, _ptr(q), q.stride(0), q.stride(1), _ptr(page_table), page_table.stride(0),
        ctypes.byref(ks), ctypes.byref(vs), float(sm_scale), _ptr(out), out.stride(0),
        out.stride(1), _ptr(lse), _stream(stream, dev)))
    return out, lse


def batch_decode_append(plan: Plan, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        page_table: torch.Tensor, k_pool: KVPool, v_pool: KVPool, sm_scale: float,
                        workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """Decode with the step's new token appended (nvfp4_batch_decode_append): k_new / v_new
    bf16 [batch, Hkv, Dk / Dv] go to token kv_len-1 of each request, then attention as
    ``batch_decode``."""
    for name, t, d in (("k_new", k_new, plan.head_dim_qk), ("v_new", v_new, plan.head_dim_vo)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(-1) != 1 \
                or tuple(t.shape) != (plan.batch, plan.num_kv_heads, d):
            raise ValueError(f"{name} must be bf16 [{plan.batch}, {plan.num_kv_heads}, {d}] "
                             "with a contiguous last dim")
    rows = _check_rows(plan, q, page_table, out, lse)
    _check_pools(plan, k_pool, v_pool)
    _check_workspace(plan, workspace)
    dev = _device(q, k_new, v_new, page_table, *k_pool.tensors(), *v_pool.tensors(), workspace,
                  out, lse)
    if out is None:
        out = torch.empty((rows, plan.num_qo_heads, plan.head_dim_vo), dtype=torch.float32,
                          device=dev)
    if lse is None:
        lse = torch.empty((rows, plan.num_qo_heads), dtype=torch.float32, device=dev)
    ks, vs = k_pool.struct(), v_pool.struct()
    args = (plan.handle, _ptr(q), q.stride(0), q.stride(1), _ptr(k_new), k_new.stride(0),
            k_new.stride(1), _ptr(v_new), v_new.stride(0), v_new.stride(1), _ptr(page_table),
            page_table.stride(0), ctypes.byref(ks), ctypes.byref(vs), float(sm_scale),
            _ptr(workspace), workspace.numel(), _ptr(out), out.stride(0), out.stride(1),
            _ptr(lse), _stream(stream, dev))
    if prepare:
        return Prepared(lib.nvfp4_batch_decode_append, args,
                        (plan, q, k_new, v_new, page_table, k_pool, v_pool, ks, vs, workspace,
                         out, lse))
    check(lib.nvfp4_batch_decode_append(*args))
    return out, lse


def kv_checksum(plan: Plan, page_table: torch.Tensor, k_pool: KVPool, v_pool: KVPool,
                workspace: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None,
                prepare: bool = False):
    """XOR checksum of the KV bytes a decode plan reads, streamed the way the decode
    kernel streams them (nvfp4_kv_checksum): int32 ``[batch, Hkv]`` holding the uint32
    words, or a ``Prepared`` call with ``prepare=True``."""
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.stride(1) != 1 \
            or page_table.shape[0] < plan.batch or page_table.shape[1] < plan.max_pages():
        raise ValueError(f"page_table must be int32 [>= {plan.batch}, >= {plan.max_pages()}] "
                         "with contiguous rows")
    _check_pools(plan, k_pool, v_pool)
    _check_workspace(plan, workspace)
    shape = (plan.batch, plan.num_kv_heads)
    if out is not None and (out.dtype != torch.int32 or tuple(out.shape) != shape
                            or not out.is_contiguous()):
        raise ValueError(f"out must be contiguous int32 of shape {shape}")
    dev = _device(page_table, *k_pool.tensors(), *v_pool.tensors(), workspace, out)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=dev)
    ks, vs = k_pool.struct(), v_pool.struct()
    args = (plan.handle, _ptr(page_table), page_table.stride(0), ctypes.byref(ks),
            ctypes.byref(vs), _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream, dev))
    if prepare:
        return Prepared(lib.nvfp4_kv_checksum, args,
                        (plan, page_table, k_pool, v_pool, ks, vs, workspace, out))
    check(lib.nvfp4_kv_checksum(*args))
    return out


def batch_prefill(plan: Plan, q: torch.Tensor, page_table: torch.Tensor, k_pool: KVPool,
                  v_pool: KVPool, sm_scale: float, workspace: torch.Tensor,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  stream=None, prepare: bool = False):
    """Prefill / extend attention; returns (O fp32 [total_q, Hq, Dv], LSE fp32 [total_q, Hq]),
    or a ``Prepared`` call with ``prepare=True``."""
    return _attn(lib.nvfp4_batch_prefill, plan, q, page_table, k_pool, v_pool, sm_scale,
                 workspace, out, lse, stream, prepare)


def batch_prefill_masked(plan: Plan, q: torch.Tensor, page_table: torch.Tensor, k_pool: KVPool,
                         v_pool: KVPool, mask: torch.Tensor, sm_scale: float,
                         workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """Prefill over the paged cache with a packed custom mask (nvfp4_batch_prefill_masked):
    ``mask`` uint8, the requests' bits one segment after the other, little-endian, each
    segment padded to a byte, and 8 more readable bytes at the end."""
    if not plan.custom_mask:
        raise ValueError("the plan was made without custom_mask")
    if mask.dtype != torch.uint8 or mask.dim() != 1 or not mask.is_contiguous() \
            or mask.numel() < plan.mask_bytes + 8:
        raise ValueError(f"mask must be a contiguous uint8 vector of at least "
                         f"{plan.mask_bytes} + 8 bytes")
    rows = _check_rows(plan, q, page_table, out, lse)
    _check_pools(plan, k_pool, v_pool)
    _check_workspace(plan, workspace)
    dev = _device(q, page_table, *k_pool.tensors(), *v_pool.tensors(), mask, workspace, out, lse)
    if out is None:
        out = torch.empty((rows, plan.num_qo_heads, plan.head_dim_vo), dtype=torch.float32,
                          device=dev)
    if lse is None:
        lse = torch.empty((rows, plan.num_qo_heads), dtype=torch.float32, device=dev)
    ks, vs = k_pool.struct(), v_pool.struct()
    args = (plan.handle, _ptr(q), q.stride(0), q.stride(1), _ptr(page_table), page_table.stride(0),
            ctypes.byref(ks), ctypes.byref(vs), _ptr(mask), float(sm_scale), _ptr(workspace),
            workspace.numel(), _ptr(out), out.stride(0), out.stride(1), _ptr(lse),
            _stream(stream, dev))
    if prepare:
        return Prepared(lib.nvfp4_batch_prefill_masked, args,
                        (plan, q, page_table, k_pool, v_pool, ks, vs, mask, workspace, out, lse))
    check(lib.nvfp4_batch_prefill_masked(*args))
    return out, lse


def batch_prefill_ragged(plan: Plan, q: torch.Tensor, k: RaggedKV, v: RaggedKV, sm_scale: float,
                         workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """Prefill over ragged K/V rows (nvfp4_batch_prefill_ragged); the plan carries the
    rows of each request (``kv_indptr``).  Returns (O, LSE) as ``batch_prefill``."""
    if not plan.ragged:
        raise ValueError("the plan was made for paged KV: create it with kv_indptr")
    rows = plan.total_rows
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.stride(-1) != 1 \
            or tuple(q.shape) != (rows, plan.num_qo_heads, plan.head_dim_qk):
        raise ValueError(f"q must be bf16 [{rows}, {plan.num_qo_heads}, {plan.head_dim_qk}] "
                         "with a contiguous last dim")
    _check_outputs(plan, out, lse)
    _check_workspace(plan, workspace)
    for name, r, d in (("k", k, plan.head_dim_qk), ("v", v, plan.head_dim_vo)):
        if r.head_dim != d or r.num_kv_heads != plan.num_kv_heads or r.dtype != plan.kv_dtype:
            raise ValueError(f"{name} is ({r.num_kv_heads} heads, dim {r.head_dim}, {r.dtype}); "
                             f"the plan needs ({plan.num_kv_heads}, {d}, {plan.kv_dtype})")
    dev = _device(q, *k.tensors(), *v.tensors(), workspace, out, lse)
    if out is None:
        out = torch.empty((rows, plan.num_qo_heads, plan.head_dim_vo), dtype=torch.float32,
                          device=dev)
    if lse is None:
        lse = torch.empty((rows, plan.num_qo_heads), dtype=torch.float32, device=dev)
    ks, vs = k.struct(), v.struct()
    args = (plan.handle, _ptr(q), q.stride(0), q.stride(1), ctypes.byref(ks), ctypes.byref(vs),
            float(sm_scale), _ptr(workspace), workspace.numel(), _ptr(out), out.stride(0),
            out.stride(1), _ptr(lse), _stream(stream, dev))
    if prepare:
        return Prepared(lib.nvfp4_batch_prefill_ragged, args,
                        (plan, q, k, v, ks, vs, workspace, out, lse))
    check(lib.nvfp4_batch_prefill_ragged(*args))
    return out, lse


def merge_partials(plan: Plan, workspace: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                   stream=None, prepare: bool = False):
    """Write the split rows of a deferred-merge run into out / lse (nvfp4_merge_partials)."""
    if out is None or lse is None:
        raise ValueError("out and lse are the run's outputs and must be given")
    _check_outputs(plan, out, lse)
    _check_workspace(plan, workspace)
    dev = _device(workspace, out, lse)
    args = (plan.handle, _ptr(workspace), workspace.numel(), _ptr(out), out.stride(0),
            out.stride(1), _ptr(lse), _stream(stream, dev))
    if prepare:
        return Prepared(lib.nvfp4_merge_partials, args, (plan, workspace, out, lse))
    check(lib.nvfp4_merge_partials(*args))
    return out, lse


def merge_states(o_parts: torch.Tensor, lse_parts: torch.Tensor, out=None, lse=None, stream=None):
    """Merge partial states: o_parts fp32 [rows, n, H, D], lse_parts fp32 [rows, n, H]
    (both contiguous); out fp32 [rows, H, D] and lse fp32 [rows, H], contiguous."""
    if o_parts.dim() != 4 or o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts must be fp32 [rows, n, H, D] and lse_parts fp32 [rows, n, H]")
    if tuple(lse_parts.shape) != tuple(o_parts.shape[:3]):
        raise ValueError(f"lse_parts must have shape {tuple(o_parts.shape[:3])}")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    rows, n, h, d = o_parts.shape
    for name, t, shape in (("out", out, (rows, h, d)), ("lse", lse, (rows, h))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous fp32 of shape {shape}")
    dev = _device(o_parts, lse_parts, out, lse)
    if out is None:
        out = torch.empty((rows, h, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((rows, h), dtype=torch.float32, device=dev)
    check(lib.nvfp4_merge_states(_ptr(o_parts), _ptr(lse_parts), rows, n, h, d, _ptr(out),
                                 _ptr(lse), _stream(stream, dev)))
    return out, lse
