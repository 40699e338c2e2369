"""GPU parity of the FP8 e4m3 KV type and of ragged (non-paged) prefill KV against the
oracle, on the same seeded inputs: the FP8 quantiser bit for bit, attention within the
parity tolerance (O max |err| <= 1e-2, LSE relative <= 1e-3, alpha in [0.99, 1.01]).

FP8 caches here hold the oracle's own bytes; pool slots no request owns hold random
bytes (NaN codes among them), and outputs start as NaN."""
import math

import numpy as np
import pytest
import torch

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import synth
from oracle import nvfp4_ref as ref
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _run(w, layout="HND", chunk=None, **kw):
    c = gh.build_oracle_case(w, layout=layout, kv_dtype="fp8", **kw)
    plan = gh.make_plan(w, chunk, kv_dtype="fp8")
    o, lse = gh.run_gpu(c, plan)
    o_ref, lse_ref = gh.oracle_reference(c)
    err = gh.assert_attention_close(o, lse, o_ref, lse_ref, w.name)
    print(f"fp8 {w.name} layout={layout} chunk={chunk}: max |O err| {err:.2e}", flush=True)
    return err, plan


@pytest.mark.parametrize("head_dim,layout,gscale", [(128, "HND", 1.0), (64, "NHD", 1.0),
                                                    (256, "HND", 0.375), (128, "NHD", 3.0)])
def test_fp8_quantize_bit_exact(head_dim, layout, gscale):
    w = synth.custom("q8", kv_lens=[1, 17, 64, 200, 33], num_kv_heads=2, head_dim_qk=head_dim,
                     seed=131)
    _, k, v = synth.draw_qkv(w)
    k = k.clone()
    # ties between e4m3 neighbours (after the scale), zeros, signed zeros, saturation,
    # subnormals
    pos = ref.e4m3_value(np.arange(127))
    ties = torch.from_numpy(((pos[40:56] + pos[41:57]) / 2) * gscale).to(torch.bfloat16)
    k[0, 0, :16] = ties
    k[1, 0, :16] = 0.0
    k[1, 1, :16] = -0.0
    k[2, 0, :16] = 1e30
    k[3, 1, :16] = -1e-30
    k[4, 0, 16:32] = torch.linspace(-2.0 ** -8, 2.0 ** -8, 16) * gscale
    pt = synth.page_table(w)
    slots = synth.token_slots(w, pt)
    pools = []
    for d in (head_dim, head_dim):
        pool = nv.KVPool.empty(w.pool_pages, 2, 16, d, layout, "cuda", global_scale=gscale,
                               dtype="fp8")
        pool.data.fill_(0xAB)
        pools.append(pool)
    nv.quantize_kv(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), pools[0], pools[1])
    torch.cuda.synchronize()
    for x, pool in ((k, pools[0]), (v, pools[1])):
        want = ref.quantize_fp8(x.double().numpy(), gscale)
        data = pool.data.cpu().numpy()
        pages, offs = slots // 16, slots % 16
        rows = data[pages, :, offs, :] if layout == "HND" else data[pages, offs, :, :]
        assert np.array_equal(rows, want)


def test_fp8_single_decode_config():
    _run(synth.workload("single_decode"), chunk=None)


@pytest.mark.parametrize("chunk", [-1, 32, 0])
def test_fp8_decode_ragged_and_split(chunk):
    w = synth.custom("d8split", kv_lens=[1, 33, 300, 1000, 77, 0], num_qo_heads=8,
                     num_kv_heads=2, seed=141)
    _run(w, chunk=chunk)


@pytest.mark.parametrize("dk,dv,hq,hkv", [(64, 64, 4, 1), (128, 64, 8, 2), (256, 128, 8, 2),
                                          (256, 256, 16, 1), (256, 64, 4, 4), (128, 128, 40, 2),
                                          (512, 256, 8, 1), (512, 128, 8, 2), (512, 64, 4, 1)])
def test_fp8_decode_head_dims_and_groups(dk, dv, hq, hkv):
    """FP8 decode at every head-dim pair; the 512-dim pairs run the register kernel at
    pages of 16 tokens (their rings do not fit the LDS)."""
    w = synth.custom(f"d8dims{dk}x{dv}", kv_lens=[150, 513, 40], num_qo_heads=hq,
                     num_kv_heads=hkv, head_dim_qk=dk, head_dim_vo=dv, seed=dk + hq)
    _run(w, chunk=64)


@pytest.mark.parametrize("layout,page_size", [("NHD", 16), ("HND", 1), ("HND", 4), ("NHD", 64)])
def test_fp8_decode_layouts_and_pages(layout, page_size):
    w = synth.custom("d8layout", kv_lens=[200, 31, 1030], num_qo_heads=32, num_kv_heads=8,
                     page_size=page_size, seed=151)
    _run(w, layout=layout, chunk=32)


@pytest.mark.parametrize("layout,page_size", [("HND", 16), ("NHD", 1)])
def test_fp8_decode_512_layouts_and_pages(layout, page_size):
    w = synth.custom("d8w512", kv_lens=[700, 17, 1500], num_qo_heads=8, num_kv_heads=1,
                     head_dim_qk=512, head_dim_vo=256, page_size=page_size, seed=153)
    _run(w, layout=layout, chunk=64)


def test_fp8_decode_global_scales_and_unequal_strides():
    w = synth.custom("d8gs", kv_lens=[90, 300], num_qo_heads=8, num_kv_heads=2, seed=161)
    _run(w, chunk=-1, k_global=0.5, v_global=2.0)
    _run(w, chunk=32, k_pad=(1, 1, 3, 16), v_pad=(2, 0, 1, 32))


def test_fp8_vones_uniform_probe():
    """Q = 0 gives uniform scores: LSE = ln(kv_len) and, with V = 1 (exact in FP8),
    O = 1 exactly (the NVFP4 probe gives 1.03125 from the block scale; FP8 has none)."""
    w = synth.custom("d8probe", kv_lens=[1, 100, 2049], num_qo_heads=4, num_kv_heads=1,
                     seed=171)
    c = gh.build_oracle_case(w, kv_dtype="fp8")
    c.q.zero_()
    c.v_pool.data.fill_(0x38)   # e4m3 0x38 = 1.0
    plan = gh.make_plan(w, 64, kv_dtype="fp8")
    o, lse = gh.run_gpu(c, plan)
    assert np.all(o == 1.0)
    for b, L in enumerate(w.kv_lens):
        assert np.allclose(lse[b], math.log(L), rtol=0, atol=1e-5)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("chunk", [-1, 64])
def test_fp8_prefill_extend(causal, chunk):
    w = synth.custom("p8ext", kv_lens=[300, 64, 1100, 17], qo_lens=[45, 64, 200, 1],
                     num_qo_heads=32, num_kv_heads=8, causal=causal, seed=181)
    _run(w, chunk=chunk)


@pytest.mark.parametrize("dk,dv,hq,hkv,page_size", [(64, 64, 4, 4, 16), (256, 128, 8, 2, 16),
                                                    (256, 256, 8, 1, 16), (128, 64, 8, 2, 1),
                                                    (256, 128, 16, 8, 1)])
def test_fp8_prefill_head_dims_and_pages(dk, dv, hq, hkv, page_size):
    w = synth.custom(f"p8dims{dk}x{dv}p{page_size}", kv_lens=[90, 200], qo_lens=[90, 37],
                     num_qo_heads=hq, num_kv_heads=hkv, head_dim_qk=dk, head_dim_vo=dv,
                     page_size=page_size, causal=True, seed=dk + page_size)
    _run(w, chunk=-1)


def test_fp8_prefill_nhd_and_unequal_strides():
    w = synth.custom("p8nhd", kv_lens=[60, 150], qo_lens=[20, 50], num_qo_heads=8,
                     num_kv_heads=2, causal=True, seed=191)
    _run(w, layout="NHD", chunk=-1)
    _run(w, chunk=32, k_pad=(1, 1, 3, 16), v_pad=(2, 0, 1, 32))


def test_fp8_checksum_is_exact():
    from tests.test_gpu_parity import _host_checksum
    w = synth.custom("cks8", kv_lens=[150, 300, 77, 0, 33, 1000], num_qo_heads=32,
                     num_kv_heads=8, seed=201)
    c = gh.build_oracle_case(w, layout="NHD", kv_dtype="fp8")
    plan = gh.make_plan(w, 16, kv_dtype="fp8")
    ws = plan.new_workspace()
    plan.upload(ws)
    got = nv.kv_checksum(plan, c.page_table, c.k_pool, c.v_pool, ws)
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            assert int(got[b, h]) == _host_checksum(c, b, h), (b, h)


# ------------------------------------------------------------------- ragged --

def _ragged_case(kv_dtype, kv_lens, qo_lens, hq, hkv, dk, dv, causal, seed, start=5):
    """Ragged rows (requests back to back from row ``start``), the rows before and after
    them random bytes and NaN scales; the oracle's own quantised bytes in between."""
    w = synth.custom("ragged", kv_lens=kv_lens, qo_lens=qo_lens, num_qo_heads=hq,
                     num_kv_heads=hkv, head_dim_qk=dk, head_dim_vo=dv, causal=causal, seed=seed)
    q, k, v = synth.draw_qkv(w)
    total = sum(kv_lens)
    rows = start + total + 15
    rng = np.random.default_rng(seed)
    kv_ind = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32) + start
    arrays = []
    for x, d in ((k, dk), (v, dv)):
        if kv_dtype == "fp8":
            data_q, sf_q = ref.quantize_fp8(x.double().numpy()), None
        else:
            data_q, sf_q = ref.quantize(x.double().numpy())
        data = rng.integers(0, 256, (rows, hkv, data_q.shape[-1]), dtype=np.uint8)
        data[start:start + total] = data_q
        sf = None
        if sf_q is not None:
            sf = np.full((rows, hkv, d // 16), synth.SF_POISON, dtype=np.uint8)
            sf[start:start + total] = sf_q
        arrays.append((data, sf))
    dev = lambda a: None if a is None else torch.from_numpy(a).cuda()
    kr = nv.RaggedKV(dev(arrays[0][0]), dev(arrays[0][1]), head_dim=dk, dtype=kv_dtype)
    vr = nv.RaggedKV(dev(arrays[1][0]), dev(arrays[1][1]), head_dim=dv, dtype=kv_dtype)
    return w, q, kr, vr, arrays, kv_ind


@pytest.mark.parametrize("kv_dtype", ["nvfp4", "fp8"])
@pytest.mark.parametrize("causal,chunk", [(True, -1), (True, 64), (False, 0)])
def test_ragged_prefill_matches_oracle(kv_dtype, causal, chunk):
    kv_lens, qo_lens = [300, 64, 1100, 17, 0], [45, 64, 200, 1, 0]
    w, q, kr, vr, arrays, kv_ind = _ragged_case(kv_dtype, kv_lens, qo_lens, 32, 8, 128, 128,
                                                causal, 211)
    plan = nv.Plan(kv_lens, qo_indptr=synth.indptr(qo_lens).tolist(), kv_indptr=kv_ind.tolist(),
                   num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, causal=causal,
                   kv_chunk_tokens=chunk, num_cus=256, kv_dtype=kv_dtype)
    ws = plan.new_workspace()
    plan.upload(ws)
    o = torch.full((w.total_q, 32, 128), float("nan"), device="cuda")
    lse = torch.full((w.total_q, 32), float("nan"), device="cuda")
    nv.batch_prefill_ragged(plan, q.cuda(), kr, vr, w.sm_scale, ws, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref.ragged_attention(q.double().numpy(), arrays[0][0], arrays[0][1],
                                          arrays[1][0], arrays[1][1], kv_ind,
                                          synth.indptr(qo_lens), w.sm_scale, causal,
                                          kv_dtype=kv_dtype)
    err = gh.assert_attention_close(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref,
                                    lse_ref, f"ragged {kv_dtype}")
    print(f"ragged {kv_dtype} causal={causal} chunk={chunk}: max |O err| {err:.2e}", flush=True)


@pytest.mark.parametrize("kv_dtype,dk,dv", [("nvfp4", 512, 256), ("nvfp4", 256, 128),
                                            ("fp8", 256, 256), ("fp8", 64, 64)])
def test_ragged_prefill_head_dims(kv_dtype, dk, dv):
    kv_lens, qo_lens = [90, 200, 33], [90, 37, 33]
    w, q, kr, vr, arrays, kv_ind = _ragged_case(kv_dtype, kv_lens, qo_lens, 8, 2, dk, dv, True,
                                                dk + dv, start=0)
    plan = nv.Plan(kv_lens, qo_indptr=synth.indptr(qo_lens).tolist(), kv_indptr=kv_ind.tolist(),
                   num_qo_heads=8, num_kv_heads=2, head_dim_qk=dk, head_dim_vo=dv, causal=True,
                   kv_chunk_tokens=-1, num_cus=256, kv_dtype=kv_dtype)
    ws = plan.new_workspace()
    plan.upload(ws)
    o, lse = nv.batch_prefill_ragged(plan, q.cuda(), kr, vr, w.sm_scale, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref.ragged_attention(q.double().numpy(), arrays[0][0], arrays[0][1],
                                          arrays[1][0], arrays[1][1], kv_ind,
                                          synth.indptr(qo_lens), w.sm_scale, True,
                                          kv_dtype=kv_dtype)
    gh.assert_attention_close(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref,
                              lse_ref, f"ragged {kv_dtype} {dk}x{dv}")
