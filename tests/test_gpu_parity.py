"""GPU parity: the HIP library against the oracle on the same seeded inputs.

The caches here are filled with the oracle's own quantised bytes (the kernels and the
reference consume the same bytes); the quantiser kernel is checked separately, bit
for bit.  Every output buffer starts as NaN, and every pool slot no request owns
holds random bytes with NaN scales, so a missed write or a stray read shows up."""
import math

import numpy as np
import pytest
import torch

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import synth
from oracle import nvfp4_ref as ref
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on CPU-only hosts)")


def _run_case(w, layout="HND", chunk=None, **kw):
    c = gh.build_oracle_case(w, layout=layout, **kw)
    plan = gh.make_plan(w, chunk)
    o, lse = gh.run_gpu(c, plan)
    o_ref, lse_ref = gh.oracle_reference(c)
    print(f"case {w.name} layout={layout} chunk={chunk} info={plan.info()}", flush=True)
    return gh.assert_attention_close(o, lse, o_ref, lse_ref, w.name), plan


# ------------------------------------------------------------------ quantiser --

@pytest.mark.parametrize("head_dim,layout,gscale", [(128, "HND", 1.0), (64, "NHD", 1.0),
                                                    (512, "HND", 1.0), (256, "HND", 0.375),
                                                    (128, "NHD", 3.0)])
def test_quantize_kv_bit_exact(head_dim, layout, gscale):
    w = synth.custom("quant", kv_lens=[1, 17, 64, 200, 33], num_kv_heads=2, head_dim_qk=head_dim,
                     seed=31)
    _, k, v = synth.draw_qkv(w)
    # adversarial rows: exact ties, zeros, huge and tiny magnitudes, negative zero
    k = k.clone()
    k[0, 0, :16] = torch.tensor([6.0, -3.0, 1.5, 0.75, -0.25, 5.0, 2.5, 1.75] * 2)
    k[1, 0, :16] = 0.0
    k[1, 1, :16] = -0.0
    k[2, 0, :16] = 1e30
    k[3, 1, :16] = 1e-30
    k[4, 0, 16:32] = torch.linspace(-2.0 ** -8, 2.0 ** -8, 16)
    pt = synth.page_table(w)
    slots = synth.token_slots(w, pt)
    dev = "cuda"
    pools = []
    for x, d in ((k, head_dim), (v, head_dim)):
        pool = nv.KVPool.empty(w.pool_pages, 2, 16, d, layout, dev, global_scale=gscale)
        pool.data.fill_(0xAB)
        pool.sf.fill_(0xCD)
        pools.append(pool)
    sl = torch.from_numpy(slots).to(dev)
    sl[3] = -1  # a skipped token
    nv.quantize_kv(k.to(dev), v.to(dev), sl, pools[0], pools[1])
    torch.cuda.synchronize()
    for x, pool in zip((k, v), pools):
        packed, sf = ref.quantize(x.double().numpy(), gscale)
        data = pool.data.cpu().numpy()
        sfs = pool.sf.cpu().numpy()
        pages, offs = slots // 16, slots % 16
        got_d = data[pages, :, offs] if layout == "HND" else data[pages, offs]
        got_s = sfs[pages, :, offs] if layout == "HND" else sfs[pages, offs]
        keep = np.ones(len(slots), bool)
        keep[3] = False
        assert np.array_equal(got_d[keep], packed[keep]), "packed bytes differ"
        assert np.array_equal(got_s[keep], sf[keep]), "scale bytes differ"
        assert np.all(got_d[3] == 0xAB) and np.all(got_s[3] == 0xCD)
        # slots nobody wrote are untouched
        written = np.zeros(data.shape[0] * 16, bool)
        written[slots[keep]] = True
        untouched = ~written.reshape(-1, 16)
        rest = data.transpose(0, 2, 1, 3)[untouched] if layout == "HND" else data[untouched]
        assert np.all(rest == 0xAB)


# ------------------------------------------------------------------- decode ----

def test_single_decode_config():
    _run_case(synth.workload("single_decode"))


@pytest.mark.parametrize("chunk", [-1, 16, 32, 48, 0])
def test_decode_ragged_and_split(chunk):
    w = synth.custom("ragged", kv_lens=[1, 15, 16, 17, 100, 300, 33, 512], num_qo_heads=8,
                     num_kv_heads=2, seed=5)
    _run_case(w, chunk=chunk)


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_decode_layouts(layout):
    w = synth.custom("layout", kv_lens=[70, 129, 5], num_qo_heads=8, num_kv_heads=4, seed=6)
    _run_case(w, layout=layout, chunk=32)


@pytest.mark.parametrize("dk,dv,hq,hkv", [(64, 64, 4, 1), (256, 128, 8, 2), (512, 256, 8, 1),
                                          (256, 256, 4, 2), (128, 64, 16, 1), (512, 128, 8, 1)])
def test_decode_head_dims(dk, dv, hq, hkv):
    w = synth.custom(f"dims{dk}x{dv}", kv_lens=[40, 97, 160], num_qo_heads=hq, num_kv_heads=hkv,
                     head_dim_qk=dk, head_dim_vo=dv, seed=dk + dv)
    _run_case(w, chunk=64)


@pytest.mark.parametrize("hq,hkv", [(1, 1), (12, 1), (16, 1), (40, 2)])
def test_decode_group_sizes(hq, hkv):
    w = synth.custom("group", kv_lens=[50, 81], num_qo_heads=hq, num_kv_heads=hkv, seed=hq)
    _run_case(w, chunk=32)


@pytest.mark.parametrize("page_size", [1, 4, 8, 32, 64])
def test_decode_page_sizes(page_size):
    w = synth.custom("pages", kv_lens=[3, 77, 130], num_qo_heads=8, num_kv_heads=2,
                     page_size=page_size, seed=page_size)
    _run_case(w, chunk=48)


def test_decode_unequal_kv_strides_and_equal_control():
    w = synth.custom("strides", kv_lens=[45, 200, 16], num_qo_heads=8, num_kv_heads=2, seed=9)
    # K and V are views of differently padded parents: genuinely different strides
    _run_case(w, k_pad=(1, 1, 3, 16), v_pad=(2, 0, 1, 32), chunk=64)
    # control: identically padded (equal, non-contiguous strides)
    _run_case(w, k_pad=(1, 1, 3, 16), v_pad=(1, 1, 3, 16), chunk=64)


def test_decode_global_scales():
    w = synth.custom("gscale", kv_lens=[64, 90], num_qo_heads=4, num_kv_heads=1, seed=12)
    _run_case(w, k_global=0.5, v_global=3.0, chunk=32)


def test_decode_empty_request_gives_zero_and_minus_inf():
    w = synth.custom("empty", kv_lens=[0, 20, 0], num_qo_heads=4, num_kv_heads=1, seed=13)
    c = gh.build_oracle_case(w)
    o, lse = gh.run_gpu(c, gh.make_plan(w, 16))
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(lse[0] == -np.inf) and np.all(lse[2] == -np.inf)
    o_ref, lse_ref = gh.oracle_reference(c)
    gh.assert_attention_close(o, lse, o_ref, lse_ref)


def test_decode_vones_uniform_probe():
    """Q = 0 and V = ones: O is exactly the dequantised one (1.03125) and LSE = ln(L)."""
    w = synth.custom("vones", kv_lens=[1, 33, 500], num_qo_heads=8, num_kv_heads=2, seed=14)
    c = gh.build_oracle_case(w)
    c.q.zero_()
    vq, vs = ref.quantize(np.ones((1, 2, 128)))
    pages, offs = synth.token_slots(w, c.pt) // 16, synth.token_slots(w, c.pt) % 16
    vd = c.v_pool.data.cpu().numpy()
    vsf = c.v_pool.sf.cpu().numpy()
    vd[pages, :, offs] = vq[0]
    vsf[pages, :, offs] = vs[0]
    c.v_pool.data.copy_(torch.from_numpy(vd))
    c.v_pool.sf.copy_(torch.from_numpy(vsf))
    o, lse = gh.run_gpu(c, gh.make_plan(w, 32))
    assert np.all(o == 1.03125)
    for b, L in enumerate(w.kv_lens):
        assert np.all(np.abs(lse[b] - math.log(L)) <= 1e-5 * max(1, math.log(L)))


def test_decode_repeat_is_bitwise_deterministic():
    w = synth.custom("repeat", kv_lens=[300, 1000], num_qo_heads=8, num_kv_heads=2, seed=15)
    c = gh.build_oracle_case(w)
    plan = gh.make_plan(w, 64)
    a = gh.run_gpu(c, plan)
    b = gh.run_gpu(c, plan)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ prefill ----

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("chunk", [-1, 64, 0])
def test_prefill_extend(causal, chunk):
    q = [1, 5, 17, 64, 130]
    prefix = [0, 3, 40, 100, 500]
    w = synth.custom("extend", kv_lens=[a + b for a, b in zip(q, prefix)], qo_lens=q,
                     num_qo_heads=8, num_kv_heads=2, causal=causal, seed=21)
    _run_case(w, chunk=chunk)


@pytest.mark.parametrize("dk,dv,hq,hkv", [(512, 256, 8, 1), (256, 128, 8, 2), (64, 64, 4, 4),
                                          (128, 128, 32, 8)])
def test_prefill_head_dims(dk, dv, hq, hkv):
    w = synth.custom(f"pdims{dk}x{dv}", kv_lens=[90, 200], qo_lens=[90, 37], num_qo_heads=hq,
                     num_kv_heads=hkv, head_dim_qk=dk, head_dim_vo=dv, causal=True, seed=dk)
    _run_case(w, chunk=-1)


@pytest.mark.parametrize("layout,page_size", [("NHD", 16), ("HND", 4), ("HND", 32)])
def test_prefill_layouts_and_pages(layout, page_size):
    w = synth.custom("playout", kv_lens=[60, 150], qo_lens=[20, 50], num_qo_heads=8,
                     num_kv_heads=2, page_size=page_size, causal=True, seed=22)
    _run_case(w, layout=layout, chunk=-1)


def test_prefill_unequal_strides():
    w = synth.custom("pstrides", kv_lens=[64, 180], qo_lens=[64, 30], num_qo_heads=8,
                     num_kv_heads=2, causal=True, seed=23)
    _run_case(w, k_pad=(1, 1, 3, 16), v_pad=(2, 0, 1, 32), chunk=-1)


def test_prefill_asym_config():
    """The asymmetric-heads causal prefill workload at its full size."""
    _run_case(synth.workload("asym_prefill"), chunk=None)


# ------------------------------------------------------------------- merge -----

def test_merge_states_matches_oracle():
    rng = np.random.default_rng(40)
    rows, n, h, d = 37, 5, 3, 128
    o_parts = rng.standard_normal((rows, n, h, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((rows, n, h)) * 3).astype(np.float32)
    lse_parts[0, :2] = -np.inf
    lse_parts[1, :] = -np.inf
    o, lse = nv.merge_states(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda())
    o_ref, lse_ref = ref.merge_states(np.moveaxis(o_parts, 1, 0), np.moveaxis(lse_parts, 1, 0))
    gh.assert_attention_close(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref)
    assert np.abs(o.cpu().numpy() - o_ref).max() < 1e-5


@pytest.mark.parametrize("decode", [True, False])
def test_deferred_merge_matches_default(decode):
    """A deferred-merge run followed by nvfp4_merge_partials writes exactly what a
    default run writes (same kernels, same order of operations)."""
    if decode:
        w = synth.custom("defer_d", kv_lens=[700, 33, 1500, 0, 260], num_qo_heads=8,
                         num_kv_heads=2, seed=31)
        chunk = 64
    else:
        w = synth.custom("defer_p", kv_lens=[300, 90], qo_lens=[40, 90], num_qo_heads=8,
                         num_kv_heads=2, causal=True, seed=32)
        chunk = 64
    c = gh.build_oracle_case(w)
    plan = gh.make_plan(w, chunk)
    assert plan.info()["num_merges"] > 0
    o_ref, lse_ref = gh.run_gpu(c, plan)
    plan2 = gh.make_plan(w, chunk)
    plan2.set_deferred_merge(True)
    ws = plan2.new_workspace(c.q.device)
    plan2.upload(ws)
    rows = c.q.shape[0]
    o = torch.full((rows, w.num_qo_heads, w.head_dim_vo), float("nan"), device=c.q.device)
    lse = torch.full((rows, w.num_qo_heads), float("nan"), device=c.q.device)
    fn = nv.batch_decode if decode else nv.batch_prefill
    fn(plan2, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o, lse=lse)
    nv.merge_partials(plan2, ws, o, lse)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o.cpu().double().numpy(), o_ref)
    np.testing.assert_array_equal(lse.cpu().double().numpy(), lse_ref)


def test_prepared_calls_match_direct_calls():
    """Prepared (pre-marshalled) quantise and decode calls launch the same work."""
    w = synth.custom("prepared", kv_lens=[300, 1200, 45], num_qo_heads=8, num_kv_heads=2, seed=33)
    c = gh.build_oracle_case(w)
    plan = gh.make_plan(w, 64)
    o_ref, lse_ref = gh.run_gpu(c, plan)
    ws = plan.new_workspace(c.q.device)
    plan.upload(ws)
    o = torch.full((w.batch, w.num_qo_heads, w.head_dim_vo), float("nan"), device=c.q.device)
    lse = torch.full((w.batch, w.num_qo_heads), float("nan"), device=c.q.device)
    call = nv.batch_decode(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o,
                           lse=lse, prepare=True)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o.cpu().double().numpy(), o_ref)
    np.testing.assert_array_equal(lse.cpu().double().numpy(), lse_ref)
    # a prepared quantise call writes the same bytes as a direct one
    src = torch.randn((4, w.num_kv_heads, w.head_dim_qk), device="cuda").bfloat16()
    slots = torch.tensor([0, 17, 33, 2], dtype=torch.int64, device="cuda")
    a = nv.KVPool.empty(4, w.num_kv_heads, 16, w.head_dim_qk)
    b = nv.KVPool.empty(4, w.num_kv_heads, 16, w.head_dim_qk)
    for p in (a, b):
        p.data.zero_()
        p.sf.zero_()
    nv.quantize_kv(src, None, slots, a, None)
    nv.quantize_kv(src, None, slots, b, None, prepare=True)()
    torch.cuda.synchronize()
    assert torch.equal(a.data, b.data) and torch.equal(a.sf, b.sf)
