"""The C-ABI library loads, exports every symbol the header declares, and rejects bad
arguments before launching anything (these run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "nvfp4_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(nvfp4_[a-z_]+)\s*\(", text)


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) == len(set(names)) == len(_lib.EXPORTS)
    assert set(names) == set(_lib.EXPORTS)
    so = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(so, n), n


def test_version_and_empty_error():
    assert "gfx950" in nv.version()
    assert nv.lib.nvfp4_last_error() is not None


def test_status_codes_match_header():
    text = open(os.path.join(ROOT, "include", "nvfp4_attn.h")).read()
    for name, code in re.findall(r"(NVFP4_(?:OK|E_[A-Z_]+))\s*=\s*(\d+)", text):
        assert _lib.STATUS[int(code)] == name


def _plan_status(**kw):
    args = dict(kv_lens=[32], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, num_cus=256)
    args.update(kw)
    try:
        nv.Plan(**args)
    except nv.NVFP4Error as e:
        return e.status, str(e)
    return "NVFP4_OK", ""


@pytest.mark.parametrize("kw,status,word", [
    (dict(num_qo_heads=6, num_kv_heads=4), "NVFP4_E_SHAPE", "multiple"),
    (dict(head_dim_qk=96), "NVFP4_E_UNSUPPORTED", "head dims"),
    (dict(head_dim_qk=128, head_dim_vo=256), "NVFP4_E_UNSUPPORTED", "vo <= qk"),
    (dict(head_dim_qk=512, head_dim_vo=512), "NVFP4_E_LDS_BUDGET", "512"),
    (dict(page_size=12), "NVFP4_E_UNSUPPORTED", "page_size"),
    (dict(kv_chunk_tokens=40), "NVFP4_E_INVALID", "multiple of 16"),
    (dict(kv_lens=[-1]), "NVFP4_E_INVALID", "negative"),
    (dict(kv_lens=[10], qo_indptr=[0, 11]), "NVFP4_E_SHAPE", "queries"),
    (dict(kv_lens=[10, 10], qo_indptr=[0, 5, 3]), "NVFP4_E_SHAPE", "non-decreasing"),
    (dict(num_qo_heads=128, num_kv_heads=1), "NVFP4_E_UNSUPPORTED", "qo heads per kv head"),
])
def test_plan_rejections(kw, status, word):
    st, msg = _plan_status(**kw)
    assert st == status and word in msg, msg


def _fake_pool(head_dim=128, page_size=16, heads=1, pages=8, sf=0x2000, data=0x1000,
               align_shift=0):
    row = head_dim // 2
    return _lib.KVPoolStruct(data + align_shift, pages * 0 + heads * page_size * row, page_size * row,
                             row, sf, heads * page_size * head_dim // 16, page_size * head_dim // 16,
                             head_dim // 16, pages, page_size, heads, head_dim, 1.0)


def _decode(plan, **over):
    args = dict(q=0x10000, q_s_row=512, q_s_head=128, pt=0x20000, pt_stride=8,
                k=_fake_pool(), v=_fake_pool(), sm=0.1, ws=0x40000,
                ws_bytes=plan.workspace_bytes, o=0x80000, o_s_row=512, o_s_head=128, lse=0x90000)
    args.update(over)
    st = nv.lib.nvfp4_batch_decode(plan.handle, args["q"], args["q_s_row"], args["q_s_head"],
                                   args["pt"], args["pt_stride"], ctypes.byref(args["k"]),
                                   ctypes.byref(args["v"]), args["sm"], args["ws"], args["ws_bytes"],
                                   args["o"], args["o_s_row"], args["o_s_head"], args["lse"], None)
    return _lib.STATUS[st], nv.lib.nvfp4_last_error().decode()


def test_run_rejections_never_launch():
    plan = nv.Plan([100], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, num_cus=256)
    cases = [
        (dict(k=_fake_pool(sf=0)), "NVFP4_E_INVALID", "scale"),
        (dict(v=_fake_pool(head_dim=64)), "NVFP4_E_SHAPE", "head_dim"),
        (dict(k=_fake_pool(page_size=32)), "NVFP4_E_SHAPE", "page_size"),
        (dict(k=_fake_pool(heads=2)), "NVFP4_E_SHAPE", "num_kv_heads"),
        (dict(k=_fake_pool(align_shift=8)), "NVFP4_E_SHAPE", "multiples"),
        (dict(q=0x10004), "NVFP4_E_SHAPE", "q rows"),
        (dict(o_s_head=130), "NVFP4_E_SHAPE", "o rows"),
        (dict(pt_stride=3), "NVFP4_E_SHAPE", "pt_stride"),
        (dict(ws=0), "NVFP4_E_WORKSPACE", "NULL"),
        (dict(ws_bytes=16), "NVFP4_E_WORKSPACE", "needs"),
        (dict(), "NVFP4_E_WORKSPACE", "uploaded"),   # never uploaded
        (dict(q=0), "NVFP4_E_INVALID", "q is NULL"),
        (dict(sm=float("nan")), "NVFP4_E_INVALID", "sm_scale"),
    ]
    for over, status, word in cases:
        st, msg = _decode(plan, **over)
        assert st == status and word in msg, (over, st, msg)


def test_prefill_plan_used_for_decode_is_rejected():
    plan = nv.Plan([100], qo_indptr=[0, 10], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128,
                   num_cus=256)
    st, msg = _decode(plan)
    assert st == "NVFP4_E_SHAPE" and "prefill" in msg


def test_merge_states_rejections():
    f = nv.lib.nvfp4_merge_states
    assert _lib.STATUS[f(0x1000, 0x2000, 4, 0, 2, 64, 0x3000, 0x4000, None)] == "NVFP4_E_INVALID"
    assert _lib.STATUS[f(0x1000, 0x2000, 4, 2, 2, 66, 0x3000, 0x4000, None)] == "NVFP4_E_UNSUPPORTED"
    assert _lib.STATUS[f(0, 0x2000, 4, 2, 2, 64, 0x3000, 0x4000, None)] == "NVFP4_E_INVALID"
    assert _lib.STATUS[f(0x1000, 0x2000, 0, 2, 2, 64, 0x3000, 0x4000, None)] == "NVFP4_OK"


def test_quantize_rejections():
    q = nv.lib.nvfp4_quantize_kv
    k = _fake_pool()
    st = q(None, 0, 0, None, 0, 0, 4, 0x5000, None, None, None)
    assert _lib.STATUS[st] == "NVFP4_E_INVALID"
    st = q(0x10000, 1024, 128, None, 0, 0, 4, 0x5000, ctypes.byref(_fake_pool(sf=0)), None, None)
    assert _lib.STATUS[st] == "NVFP4_E_INVALID"
    st = q(0x10002, 1024, 128, None, 0, 0, 4, 0x5000, ctypes.byref(k), None, None)
    assert _lib.STATUS[st] == "NVFP4_E_SHAPE"
    st = q(0x10000, 1024, 128, None, 0, 0, 0, 0, ctypes.byref(k), None, None)
    assert _lib.STATUS[st] == "NVFP4_OK"   # zero tokens: nothing to do


def test_deferred_merge_entry_points():
    f = nv.lib.nvfp4_merge_partials
    assert _lib.STATUS[nv.lib.nvfp4_plan_set_deferred_merge(None, 1)] == "NVFP4_E_INVALID"
    assert _lib.STATUS[f(None, 0x4000, 1 << 20, 0x8000, 512, 128, 0x9000, None)] == "NVFP4_E_INVALID"
    split = nv.Plan([3000], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, kv_chunk_tokens=64,
                    num_cus=256)
    split.set_deferred_merge(True)
    assert split.info()["num_merges"] == 1
    # the plan was never uploaded to this workspace: rejected before any launch
    st = f(split.handle, 0x40000, split.workspace_bytes, 0x80000, 512, 128, 0x90000, None)
    assert _lib.STATUS[st] == "NVFP4_E_WORKSPACE" and "uploaded" in nv.lib.nvfp4_last_error().decode()
    st = f(split.handle, 0x40000, 16, 0x80000, 512, 128, 0x90000, None)
    assert _lib.STATUS[st] == "NVFP4_E_WORKSPACE"
    # nothing split: nothing to do
    whole = nv.Plan([3000], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, kv_chunk_tokens=-1,
                    num_cus=256)
    assert _lib.STATUS[f(whole.handle, 0, 0, 0, 0, 0, 0, None)] == "NVFP4_OK"


def test_decode_append_rejections_never_launch():
    f = nv.lib.nvfp4_batch_decode_append

    def call(plan, k_new=0x50000, v_new=0x60000, kn_s=(256, 128), **over):
        args = dict(q=0x10000, pt=0x20000, pt_stride=8, k=_fake_pool(), v=_fake_pool(), ws=0x40000)
        args.update(over)
        st = f(plan.handle, args["q"], 512, 128, k_new, kn_s[0], kn_s[1], v_new, 256, 128,
               args["pt"], args["pt_stride"], ctypes.byref(args["k"]), ctypes.byref(args["v"]),
               0.1, args["ws"], plan.workspace_bytes, 0x80000, 512, 128, 0x90000, None)
        return _lib.STATUS[st], nv.lib.nvfp4_last_error().decode()

    plan = nv.Plan([100], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, num_cus=256)
    assert call(plan, k_new=0)[0] == "NVFP4_E_INVALID"
    st, msg = call(plan, v_new=0x60002)
    assert st == "NVFP4_E_SHAPE" and "v_new" in msg
    st, msg = call(plan, kn_s=(250, 128))
    assert st == "NVFP4_E_SHAPE" and "k_new" in msg
    st, msg = call(plan)  # valid rows: the usual decode checks follow (never uploaded)
    assert st == "NVFP4_E_WORKSPACE" and "uploaded" in msg
    small = nv.Plan([100], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, page_size=8,
                    num_cus=256)
    st, msg = call(small, k=_fake_pool(page_size=8), v=_fake_pool(page_size=8))
    assert st == "NVFP4_E_UNSUPPORTED" and "page_size" in msg
    prefill = nv.Plan([100], qo_indptr=[0, 10], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128,
                      num_cus=256)
    st, msg = call(prefill)
    assert st == "NVFP4_E_SHAPE" and "prefill" in msg


def test_binding_checks_shapes_against_the_plan():
    """The C library takes pointers; the binding rejects tensors that do not cover the
    plan's rows before any launch."""
    import torch
    plan = nv.Plan([100, 30], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, num_cus=256)
    pt = torch.zeros((2, 8), dtype=torch.int32)
    pool = nv.KVPool.empty(16, 1, 16, 128, device="cpu")
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8)
    bad_q = torch.zeros((1, 4, 128), dtype=torch.bfloat16)           # one request short
    with pytest.raises(ValueError, match="q must be"):
        nv.batch_decode(plan, bad_q, pt, pool, pool, 0.1, ws)
    q = torch.zeros((2, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="page_table"):
        nv.batch_decode(plan, q, pt[:1], pool, pool, 0.1, ws)
    with pytest.raises(ValueError, match="out must"):
        nv.batch_decode(plan, q, pt, pool, pool, 0.1, ws, out=torch.zeros((2, 4, 64)))
    kn = torch.zeros((2, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="v_new"):
        nv.batch_decode_append(plan, q, kn, kn[:1], pt, pool, pool, 0.1, ws)


def test_lds_budget_is_computed_and_rejects_what_does_not_fit():
    """The plan's on-chip check uses the kernels' own LDS footprint: the 512/512 prefill
    tile needs more LDS than a CU has and is refused as such; every supported pair of
    head dims fits at every page size."""
    st, msg = _plan_status(kv_lens=[64], qo_indptr=[0, 8], head_dim_qk=512, head_dim_vo=512)
    assert st == "NVFP4_E_LDS_BUDGET" and "LDS" in msg and "163840" in msg, msg
    st, msg = _plan_status(kv_lens=[64], head_dim_qk=512, head_dim_vo=512)
    assert st == "NVFP4_E_LDS_BUDGET", msg
    for dk in (64, 128, 256, 512):
        for dv in (64, 128, 256, 512):
            if dv > dk or (dk, dv) == (512, 512):
                continue
            for ps in (1, 4, 16, 64):
                for ind in (None, [0, 8]):
                    st, msg = _plan_status(kv_lens=[64], qo_indptr=ind, head_dim_qk=dk,
                                           head_dim_vo=dv, page_size=ps, num_qo_heads=8,
                                           num_kv_heads=1)
                    assert st == "NVFP4_OK", (dk, dv, ps, ind, msg)


def test_binding_refuses_host_tensors_before_any_call():
    """Tensors with the right shapes but on the host would hand host pointers to the
    kernels; the binding refuses them (and mixed devices) before calling the library."""
    import torch
    plan = nv.Plan([100, 30], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, num_cus=256)
    pt = torch.zeros((2, 8), dtype=torch.int32)
    pool = nv.KVPool.empty(16, 1, 16, 128, device="cpu")
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8)
    q = torch.zeros((2, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        nv.batch_decode(plan, q, pt, pool, pool, 0.1, ws)
    kn = torch.zeros((2, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        nv.batch_decode_append(plan, q, kn, kn, pt, pool, pool, 0.1, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        plan.upload(ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        nv.quantize_kv(kn[0:1].expand(3, 1, 128).contiguous(), None,
                       torch.zeros(3, dtype=torch.int64), pool, None)
    o = torch.zeros((2, 4, 128))
    lse = torch.zeros((2, 4))
    with pytest.raises(ValueError, match="GPU tensor"):
        nv.merge_partials(plan, ws, o, lse)
    with pytest.raises(ValueError, match="GPU tensor"):
        nv.merge_states(torch.zeros((2, 3, 4, 64)), torch.zeros((2, 3, 4)))
    # a pool whose heads or dims do not match the plan
    pool64 = nv.KVPool.empty(16, 1, 16, 64, device="cpu")
    with pytest.raises(ValueError, match="k_pool"):
        nv.batch_decode(plan, q, pt, pool64, pool, 0.1, ws)
    # a page table with too few columns for the longest request (100 keys: 7 pages)
    with pytest.raises(ValueError, match="page_table"):
        nv.batch_decode(plan, q, pt[:, :6], pool, pool, 0.1, ws)
    with pytest.raises(ValueError, match="workspace"):
        nv.batch_decode(plan, q, pt, pool, pool, 0.1, ws[:8])


def test_binding_checks_sources_and_merge_shapes():
    """Sources must match their pools, and merge inputs / outputs their shapes and
    dtype, or the kernels would read or write past the buffers."""
    import torch
    kp = nv.KVPool.empty(16, 2, 16, 128, device="cpu")
    vp = nv.KVPool.empty(16, 2, 16, 64, device="cpu")
    slots = torch.zeros(5, dtype=torch.int64)
    k = torch.zeros((5, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="v must have shape"):
        nv.quantize_kv(k, torch.zeros((4, 2, 64), dtype=torch.bfloat16), slots, kp, vp)
    with pytest.raises(ValueError, match="v must have shape"):
        nv.quantize_kv(k, torch.zeros((5, 2, 128), dtype=torch.bfloat16), slots, kp, vp)
    with pytest.raises(ValueError, match="k must have shape"):
        nv.quantize_kv(torch.zeros((5, 1, 128), dtype=torch.bfloat16), None, slots, kp, None)
    with pytest.raises(ValueError, match="slot_mapping"):
        nv.quantize_kv(k, None, slots[:4], kp, None)
    with pytest.raises(ValueError, match="pool"):
        nv.quantize_kv(k, None, slots, None, None)
    o_parts = torch.zeros((2, 3, 4, 64))
    with pytest.raises(ValueError, match="fp32"):
        nv.merge_states(o_parts.double(), torch.zeros((2, 3, 4)))
    with pytest.raises(ValueError, match="lse_parts must have shape"):
        nv.merge_states(o_parts, torch.zeros((2, 3, 5)))
    with pytest.raises(ValueError, match="out must be"):
        nv.merge_states(o_parts, torch.zeros((2, 3, 4)), out=torch.zeros((2, 4, 32)))
    with pytest.raises(ValueError, match="lse must be"):
        nv.merge_states(o_parts, torch.zeros((2, 3, 4)), lse=torch.zeros((4, 2)).t())
    plan = nv.Plan([3000], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, kv_chunk_tokens=64,
                   num_cus=256)
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out must have shape"):
        nv.merge_partials(plan, ws, torch.zeros((2, 4, 128)), torch.zeros((1, 4)))
    with pytest.raises(ValueError, match="lse must"):
        nv.merge_partials(plan, ws, torch.zeros((1, 4, 128)), torch.zeros((1, 4), dtype=torch.float64))


def test_noalloc_decode_rejects_plans_beyond_its_scratch():
    """The allocation-free decode has a fixed 32 MiB scratch: a plan that needs more is
    refused, by name, before anything touches a device."""
    big = nv.Plan([8192] * 64, num_qo_heads=64, num_kv_heads=4, head_dim_qk=256,
                  kv_chunk_tokens=16, num_cus=256)
    assert big.workspace_bytes > 32 << 20
    pool = _fake_pool(head_dim=256, heads=4, pages=40000)
    st = nv.lib.nvfp4_batch_decode_noalloc(big.handle, ctypes.c_void_p(0x1000), 64 * 256, 256,
                                           ctypes.c_void_p(0x2000), 512, ctypes.byref(pool),
                                           ctypes.byref(pool), 0.1, ctypes.c_void_p(0x3000),
                                           64 * 256, 256, ctypes.c_void_p(0x4000), None)
    assert _lib.STATUS[st] == "NVFP4_E_WORKSPACE"
    msg = nv.lib.nvfp4_last_error().decode()
    assert "allocation-free" in msg and str(32 << 20) in msg


def _plan_ex_status(kv_dtype=0, kv_indptr=None, custom_mask=False, **kw):
    args = dict(kv_lens=[64], qo_indptr=[0, 8], num_qo_heads=8, num_kv_heads=1, head_dim_qk=128,
                head_dim_vo=128, num_cus=256, kv_dtype=["nvfp4", "fp8"][kv_dtype],
                kv_indptr=kv_indptr, custom_mask=custom_mask)
    args.update(kw)
    try:
        nv.Plan(**args)
    except nv.NVFP4Error as e:
        return e.status, str(e)
    return "NVFP4_OK", ""


def test_fp8_plans_price_the_tile_in_lds():
    """FP8 rows are twice as long: the 512/256 FP8 prefill tile needs more LDS than a CU
    has and is refused by the computed budget; FP8 prefill kernels exist for head dims
    up to 256.  FP8 decode covers the 512-dim pairs with the register kernel (priced by
    its exchange buffer), and the checksum, which streams through the rings, refuses
    them."""
    st, msg = _plan_ex_status(1, head_dim_qk=512, head_dim_vo=256)
    assert st == "NVFP4_E_LDS_BUDGET" and "LDS" in msg, msg
    st, msg = _plan_ex_status(1, head_dim_qk=512, head_dim_vo=128)
    assert st == "NVFP4_E_UNSUPPORTED" and "FP8" in msg, msg
    for dv in (64, 128, 256):
        for ps in (1, 16):
            st, msg = _plan_ex_status(1, qo_indptr=None, head_dim_qk=512, head_dim_vo=dv,
                                      page_size=ps)
            assert st == "NVFP4_OK", (dv, ps, msg)
    plan = nv.Plan([64], num_qo_heads=8, num_kv_heads=1, head_dim_qk=512, head_dim_vo=256,
                   num_cus=256, kv_dtype="fp8")
    st = nv.lib.nvfp4_kv_checksum(plan.handle, ctypes.c_void_p(0x4000), 64, None, None,
                                  ctypes.c_void_p(0x8000), 1 << 20, ctypes.c_void_p(0x9000),
                                  None)
    assert _lib.STATUS[st] == "NVFP4_E_UNSUPPORTED", nv.lib.nvfp4_last_error().decode()
    assert "rings" in nv.lib.nvfp4_last_error().decode()
    for dk, dv in ((64, 64), (128, 64), (128, 128), (256, 64), (256, 128), (256, 256)):
        for ind in (None, [0, 8]):
            for ps in (1, 16):
                st, msg = _plan_ex_status(1, qo_indptr=ind, head_dim_qk=dk, head_dim_vo=dv,
                                          page_size=ps)
                assert st == "NVFP4_OK", (dk, dv, ind, ps, msg)


def test_fp8_pool_rules_and_dtype_mismatch():
    plan8 = nv.Plan([100], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, num_cus=256,
                    kv_dtype="fp8")
    plan4 = nv.Plan([100], num_qo_heads=4, num_kv_heads=1, head_dim_qk=128, num_cus=256)
    fp8 = _fake_pool()
    fp8.kv_dtype = 1
    fp8.stride_page, fp8.stride_token = 16 * 128, 128
    st, msg = _decode(plan8, k=fp8, v=fp8)       # a stray scale pointer on an FP8 pool
    assert st == "NVFP4_E_INVALID" and "FP8 pool" in msg, msg
    fp8.sf = None
    st, msg = _decode(plan4, k=fp8, v=fp8)       # an FP8 pool under an NVFP4 plan
    assert st == "NVFP4_E_SHAPE" and "kv_dtype" in msg, msg
    st, msg = _decode(plan8, k=_fake_pool(), v=_fake_pool())   # NVFP4 pools, FP8 plan
    assert st == "NVFP4_E_SHAPE", msg
    # the in-launch append writes NVFP4 only
    st = nv.lib.nvfp4_batch_decode_append(plan8.handle, ctypes.c_void_p(0x10000), 512, 128,
                                          ctypes.c_void_p(0x10000), 128, 128,
                                          ctypes.c_void_p(0x10000), 128, 128,
                                          ctypes.c_void_p(0x20000), 8, ctypes.byref(fp8),
                                          ctypes.byref(fp8), 0.1, ctypes.c_void_p(0x40000),
                                          plan8.workspace_bytes, ctypes.c_void_p(0x80000), 512,
                                          128, ctypes.c_void_p(0x90000), None)
    assert _lib.STATUS[st] == "NVFP4_E_UNSUPPORTED" and "FP8" in nv.lib.nvfp4_last_error().decode()


def test_ragged_plan_rules():
    st, msg = _plan_ex_status(kv_indptr=[0, 64], qo_indptr=None)
    assert st == "NVFP4_E_SHAPE" and "qo_indptr" in msg
    st, msg = _plan_ex_status(kv_indptr=[3, 60])          # 57 rows, kv_lens says 64
    assert st == "NVFP4_E_SHAPE" and "kv_indptr" in msg
    assert _plan_ex_status(kv_indptr=[5, 69])[0] == "NVFP4_OK"
    import torch
    ragged = nv.Plan([64, 20], qo_indptr=[0, 8, 28], kv_indptr=[5, 69, 89], num_qo_heads=8,
                     num_kv_heads=1, head_dim_qk=128, num_cus=256)
    paged = nv.Plan([64, 20], qo_indptr=[0, 8, 28], num_qo_heads=8, num_kv_heads=1,
                    head_dim_qk=128, num_cus=256)
    # a ragged plan through the paged entry point and the reverse, before any launch
    st = nv.lib.nvfp4_batch_prefill(ragged.handle, ctypes.c_void_p(0x10000), 1024, 128,
                                    ctypes.c_void_p(0x20000), 8, ctypes.byref(_fake_pool()),
                                    ctypes.byref(_fake_pool()), 0.1, ctypes.c_void_p(0x40000),
                                    ragged.workspace_bytes, ctypes.c_void_p(0x80000), 1024, 128,
                                    ctypes.c_void_p(0x90000), None)
    assert _lib.STATUS[st] == "NVFP4_E_SHAPE" and "ragged" in nv.lib.nvfp4_last_error().decode()

    def rows(n, dtype=0):
        return _lib.KVRaggedStruct(0x100000, 64, 64, 0x200000, 8, 8, n, 1, 128, 1.0, dtype)
    call = lambda plan, k, v: nv.lib.nvfp4_batch_prefill_ragged(
        plan.handle, ctypes.c_void_p(0x10000), 1024, 128, ctypes.byref(k), ctypes.byref(v), 0.1,
        ctypes.c_void_p(0x40000), plan.workspace_bytes, ctypes.c_void_p(0x80000), 1024, 128,
        ctypes.c_void_p(0x90000), None)
    st = call(paged, rows(200), rows(200))
    assert _lib.STATUS[st] == "NVFP4_E_SHAPE" and "paged" in nv.lib.nvfp4_last_error().decode()
    # request 1 ends at row 89; its 16-row pages read rows up to 69 + 32 = 101
    st = call(ragged, rows(100), rows(200))
    assert _lib.STATUS[st] == "NVFP4_E_SHAPE" and "101" in nv.lib.nvfp4_last_error().decode()
    st = call(ragged, rows(101), rows(101, dtype=1))      # V says FP8, the plan NVFP4
    assert _lib.STATUS[st] in ("NVFP4_E_SHAPE", "NVFP4_E_INVALID")
    # the binding refuses host tensors and a paged plan
    k = nv.RaggedKV.empty(89, 1, 128, device="cpu")
    q = torch.zeros((28, 8, 128), dtype=torch.bfloat16)
    ws = torch.zeros(ragged.workspace_bytes, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        nv.batch_prefill_ragged(ragged, q, k, k, 0.1, ws)
    with pytest.raises(ValueError, match="paged"):
        nv.batch_prefill_ragged(paged, q, k, k, 0.1, ws)


def test_custom_mask_plan_rules():
    st, msg = _plan_ex_status(custom_mask=True, qo_indptr=None)
    assert st == "NVFP4_E_SHAPE" and "prefill" in msg, msg
    st, msg = _plan_ex_status(custom_mask=True, kv_indptr=[0, 64])
    assert st == "NVFP4_E_UNSUPPORTED" and "ragged" in msg, msg
    import torch
    plan = nv.Plan([64, 20, 5], qo_indptr=[0, 8, 28, 28], num_qo_heads=8, num_kv_heads=1,
                   head_dim_qk=128, num_cus=256, custom_mask=True, causal=True)
    assert plan.mask_bytes == (8 * 64 + 7) // 8 + (20 * 20 + 7) // 8 + 0
    # a mask plan through the unmasked entry point, and no mask given
    st = nv.lib.nvfp4_batch_prefill(plan.handle, ctypes.c_void_p(0x10000), 1024, 128,
                                    ctypes.c_void_p(0x20000), 8, ctypes.byref(_fake_pool()),
                                    ctypes.byref(_fake_pool()), 0.1, ctypes.c_void_p(0x40000),
                                    plan.workspace_bytes, ctypes.c_void_p(0x80000), 1024, 128,
                                    ctypes.c_void_p(0x90000), None)
    assert _lib.STATUS[st] == "NVFP4_E_SHAPE" and "custom mask" in nv.lib.nvfp4_last_error().decode()
    st = nv.lib.nvfp4_batch_prefill_masked(plan.handle, ctypes.c_void_p(0x10000), 1024, 128,
                                           ctypes.c_void_p(0x20000), 8,
                                           ctypes.byref(_fake_pool()), ctypes.byref(_fake_pool()),
                                           None, 0.1, ctypes.c_void_p(0x40000),
                                           plan.workspace_bytes, ctypes.c_void_p(0x80000), 1024,
                                           128, ctypes.c_void_p(0x90000), None)
    assert _lib.STATUS[st] == "NVFP4_E_INVALID" and "mask" in nv.lib.nvfp4_last_error().decode()
    unmasked = nv.Plan([64], qo_indptr=[0, 8], num_qo_heads=8, num_kv_heads=1, head_dim_qk=128,
                       num_cus=256)
    st = nv.lib.nvfp4_batch_prefill_masked(unmasked.handle, ctypes.c_void_p(0x10000), 1024, 128,
                                           ctypes.c_void_p(0x20000), 8,
                                           ctypes.byref(_fake_pool()), ctypes.byref(_fake_pool()),
                                           ctypes.c_void_p(0x50000), 0.1,
                                           ctypes.c_void_p(0x40000), unmasked.workspace_bytes,
                                           ctypes.c_void_p(0x80000), 1024, 128,
                                           ctypes.c_void_p(0x90000), None)
    assert _lib.STATUS[st] == "NVFP4_E_SHAPE"
    # the binding checks the buffer holds the bits plus 8 bytes of read-ahead
    q = torch.zeros((28, 8, 128), dtype=torch.bfloat16)
    pt = torch.zeros((3, 4), dtype=torch.int32)
    pool = nv.KVPool.empty(16, 1, 16, 128, device="cpu")
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8)
    short = torch.zeros(plan.mask_bytes + 7, dtype=torch.uint8)
    with pytest.raises(ValueError, match=r"\+ 8"):
        nv.batch_prefill_masked(plan, q, pt, pool, pool, short, 0.1, ws)
    with pytest.raises(ValueError, match="custom mask"):
        nv.batch_prefill(plan, q, pt, pool, pool, 0.1, ws)


def test_rope_plan_rules():
    """In-kernel RoPE: prefill plans only (paged or ragged), not with a custom mask, a
    positive finite base and scale, positions below 2^24; every supported shape's rotary
    tile fits the LDS budget."""
    st, msg = _plan_ex_status(qo_indptr=None, rope_theta=1e4)
    assert st == "NVFP4_E_UNSUPPORTED" and "prefill" in msg, msg
    st, msg = _plan_ex_status(custom_mask=True, rope_theta=1e4)
    assert st == "NVFP4_E_UNSUPPORTED" and "custom mask" in msg, msg
    for theta, scale in ((0.0, 1.0), (-5.0, 1.0), (float("nan"), 1.0), (float("inf"), 1.0),
                         (1e4, 0.0), (1e4, float("inf"))):
        st, msg = _plan_ex_status(rope_theta=theta, rope_scale=scale)
        assert st == "NVFP4_E_INVALID" and "rope_theta" in msg, (theta, scale, msg)
    st, msg = _plan_ex_status(kv_lens=[(1 << 24) + 1], qo_indptr=[0, 4], rope_theta=1e4)
    assert st == "NVFP4_E_UNSUPPORTED" and "2^24" in msg, msg
    assert _plan_ex_status(kv_lens=[1 << 24], qo_indptr=[0, 4], rope_theta=1e4)[0] == "NVFP4_OK"
    assert _plan_ex_status(kv_indptr=[0, 64], rope_theta=1e4, kv_dtype=1)[0] == "NVFP4_OK"
    # an unknown position encoding through the C struct
    opts = _lib.PlanOptionsStruct(0, None, 0, 7, 1e4, 1.0)
    kv = np.array([64], dtype=np.int32)
    ind = np.array([0, 8], dtype=np.int32)
    h = ctypes.c_void_p()
    st = nv.lib.nvfp4_plan_create_ex(kv.ctypes.data_as(ctypes.c_void_p),
                                     ind.ctypes.data_as(ctypes.c_void_p), 1, 8, 1, 128, 128, 16,
                                     1, 0, 256, ctypes.byref(opts), ctypes.byref(h))
    assert _lib.STATUS[st] == "NVFP4_E_INVALID" and "pos_encoding" in nv.lib.nvfp4_last_error().decode()
    # the frequency table rides in the uploaded part of the workspace: DK/2 float pairs
    plain = nv.Plan([64], qo_indptr=[0, 8], num_qo_heads=8, num_kv_heads=1, head_dim_qk=512,
                    head_dim_vo=256, num_cus=256)
    rope = nv.Plan([64], qo_indptr=[0, 8], num_qo_heads=8, num_kv_heads=1, head_dim_qk=512,
                   head_dim_vo=256, num_cus=256, rope_theta=1e4)
    assert rope.workspace_bytes == plain.workspace_bytes + 512 * 4
    for dk in (64, 128, 256, 512):
        for dv in (64, 128, 256):
            if dv > dk:
                continue
            for ps in (1, 16):
                st, msg = _plan_ex_status(page_size=ps, head_dim_qk=dk, head_dim_vo=dv,
                                          rope_theta=5e5, rope_scale=8.0)
                assert st == "NVFP4_OK", (dk, dv, ps, msg)
