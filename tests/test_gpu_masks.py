"""GPU parity of prefill with packed custom masks against the oracle (the bidirectional,
multimodal-prefix masks of the pages and random ones), over the cooperative kernel
(one to three blocks of 64 tile queries, the 512-dim wide kernel, FP8) and the register
kernel (page size 4), unsplit and split.  The 8 bytes read past the last segment hold
0xFF, so a stray bit read would show as a visible key."""
import numpy as np
import pytest
import torch

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import synth
from oracle import nvfp4_ref as ref
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _masks(kind, qo, kv, rng):
    out = []
    for q, L in zip(qo, kv):
        if kind == "random":
            m = rng.random((q, L)) < 0.55
            if q > 2:
                m[1] = False                     # a row that sees nothing
        elif kind == "prefix":
            # image prefix of the new tokens attended bidirectionally, the rest causal
            # (bottom-right aligned over the cached prefix)
            prefix = L - q
            img = max(1, q // 3)
            i = np.arange(q)[:, None]
            j = np.arange(L)[None, :]
            causal = j <= i + prefix
            both_img = (i < img) & (j >= prefix) & (j < prefix + img)
            m = causal | both_img
        else:                                    # the causal pattern itself
            m = np.arange(L)[None, :] <= np.arange(q)[:, None] + (L - q)
        out.append(m)
    return out


def _run_masked(w, masks, chunk, kv_dtype="nvfp4", causal_reference=False):
    c = gh.build_oracle_case(w, kv_dtype=kv_dtype)
    plan = nv.Plan(w.kv_lens, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                   head_dim_qk=w.head_dim_qk, head_dim_vo=w.head_dim_vo, page_size=w.page_size,
                   qo_indptr=synth.indptr(w.qo_lens).tolist(), causal=True,
                   kv_chunk_tokens=chunk, num_cus=256, kv_dtype=kv_dtype, custom_mask=True)
    packed = ref.pack_masks(masks)
    assert packed.size == plan.mask_bytes
    buf = np.concatenate([packed, np.full(8, 0xFF, dtype=np.uint8)])
    mask = torch.from_numpy(buf).cuda()
    ws = plan.new_workspace()
    plan.upload(ws)
    rows = c.q.shape[0]
    o = torch.full((rows, w.num_qo_heads, w.head_dim_vo), float("nan"), device="cuda")
    lse = torch.full((rows, w.num_qo_heads), float("nan"), device="cuda")
    nv.batch_prefill_masked(plan, c.q, c.page_table, c.k_pool, c.v_pool, mask, w.sm_scale, ws,
                            out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    o_ref, lse_ref = ref.paged_attention(c.q_np, c.k_np[0], c.k_np[1], c.v_np[0], c.v_np[1],
                                         c.pt, w.kv_lens, synth.indptr(w.qo_lens), w.page_size,
                                         w.sm_scale, False, c.layout, kv_dtype=kv_dtype,
                                         custom_mask=packed)
    err = gh.assert_attention_close(o, lse, o_ref, lse_ref, w.name)
    print(f"mask {w.name} chunk={chunk} {kv_dtype}: max |O err| {err:.2e}", flush=True)
    if causal_reference:
        o_c, lse_c = gh.oracle_reference(c)      # the same inputs with causal = True
        gh.assert_attention_close(o, lse, o_c, lse_c, w.name + " vs causal")
    return plan


@pytest.mark.parametrize("kind", ["random", "prefix"])
@pytest.mark.parametrize("chunk", [-1, 64])
def test_masked_prefill_extend(kind, chunk):
    rng = np.random.default_rng(7 if kind == "random" else 8)
    kv, qo = [300, 64, 1100, 17, 0], [45, 64, 200, 1, 0]
    w = synth.custom("mext", kv_lens=kv, qo_lens=qo, num_qo_heads=32, num_kv_heads=8,
                     causal=True, seed=221)
    _run_masked(w, _masks(kind, qo, kv, rng), chunk)


def test_causal_pattern_as_mask_equals_causal():
    kv, qo = [300, 129, 77], [45, 129, 5]
    w = synth.custom("mcausal", kv_lens=kv, qo_lens=qo, num_qo_heads=8, num_kv_heads=2,
                     causal=True, seed=222)
    _run_masked(w, _masks("causal", qo, kv, None), -1, causal_reference=True)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (40, 2)])
def test_masked_query_blocks(hq, hkv):
    """One kv head per qo head makes a tile 192 queries (three blocks of 64 lanes);
    two per qo head 96; 20 per head 9."""
    rng = np.random.default_rng(hq)
    kv, qo = [400, 250], [400, 130]
    w = synth.custom(f"mblk{hq}", kv_lens=kv, qo_lens=qo, num_qo_heads=hq, num_kv_heads=hkv,
                     causal=True, seed=223 + hq)
    _run_masked(w, _masks("random", qo, kv, rng), 128)


@pytest.mark.parametrize("dk,dv,kv_dtype,page_size", [(512, 256, "nvfp4", 16),
                                                      (256, 128, "fp8", 16),
                                                      (128, 128, "nvfp4", 4),
                                                      (64, 64, "fp8", 1)])
def test_masked_head_dims_types_and_register_kernel(dk, dv, kv_dtype, page_size):
    rng = np.random.default_rng(dk + page_size)
    kv, qo = [200, 90, 33], [70, 90, 3]
    w = synth.custom(f"mdims{dk}", kv_lens=kv, qo_lens=qo, num_qo_heads=8, num_kv_heads=1,
                     head_dim_qk=dk, head_dim_vo=dv, page_size=page_size, causal=True,
                     seed=224 + dk)
    for kind in ("random", "prefix"):
        _run_masked(w, _masks(kind, qo, kv, rng), -1, kv_dtype=kv_dtype)
