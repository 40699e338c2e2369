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


@pytest.mark.parametrize("layout,page_size", [("NHD", 16), ("HND", 4), ("NHD", 1)])
def test_decode_xcd_grouped_items(layout, page_size):
    """Pools whose kv heads sit at a short stride (NHD pages, small pages) run the work
    items XCD-grouped: each full run of 64 workgroups is permuted.  Hundreds of items
    (16-key chunks over ragged requests), so several full runs and a partial one."""
    w = synth.custom(f"xcd{layout}{page_size}", kv_lens=[1000, 777, 1500, 64, 1203, 9],
                     num_qo_heads=32, num_kv_heads=8, page_size=page_size, seed=81)
    _, plan = _run_case(w, layout=layout, chunk=16)
    assert plan.info()["num_work_items"] > 3 * 64


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


def test_prefill_request_without_queries():
    """A request with keys but no queries inside a ragged prefill batch."""
    w = synth.custom("noq", kv_lens=[40, 120, 75], qo_lens=[10, 0, 75], num_qo_heads=8,
                     num_kv_heads=2, causal=True, seed=24)
    _run_case(w, chunk=-1)
    _run_case(w, chunk=32)


@pytest.mark.parametrize("dk,chunk", [(128, -1), (128, 64), (64, -1), (256, -1), (512, -1)])
def test_prefill_vones_uniform_probe(dk, chunk):
    """Q = 0 and V = ones in a causal extend: every row's O is exactly the dequantised
    one (1.03125) and its LSE is ln of its visible keys, i + 1 + L - q for query i."""
    q = [3, 40, 100]
    prefix = [0, 17, 260]
    w = synth.custom(f"pvones{dk}", kv_lens=[a + b for a, b in zip(q, prefix)], qo_lens=q,
                     num_qo_heads=8, num_kv_heads=2, head_dim_qk=dk,
                     head_dim_vo=min(dk, 256), causal=True, seed=25)
    c = gh.build_oracle_case(w)
    c.q.zero_()
    dv = w.head_dim_vo
    vq, vs = ref.quantize(np.ones((1, 2, dv)))
    slots = synth.token_slots(w, c.pt)
    pages, offs = slots // 16, slots % 16
    vd = c.v_pool.data.cpu().numpy()
    vsf = c.v_pool.sf.cpu().numpy()
    vd[pages, :, offs] = vq[0]
    vsf[pages, :, offs] = vs[0]
    c.v_pool.data.copy_(torch.from_numpy(vd))
    c.v_pool.sf.copy_(torch.from_numpy(vsf))
    o, lse = gh.run_gpu(c, gh.make_plan(w, chunk))
    if chunk == -1:
        assert np.all(o == 1.03125)
    else:
        # split rows pass through the LSE merge, whose fp32 weights are not exact
        dev = np.abs(o - 1.03125).max()
        print(f"merged rows: max |O - 1.03125| = {dev:.3e}", flush=True)
        assert dev <= 8 * 2.0 ** -23
    row = 0
    for b, (qb, L) in enumerate(zip(q, w.kv_lens)):
        for i in range(qb):
            want = math.log(i + 1 + L - qb)
            assert np.all(np.abs(lse[row] - want) <= 1e-5 * max(1.0, want)), (b, i)
            row += 1


@pytest.mark.parametrize("dk,dv,hq,hkv", [(512, 256, 8, 1), (256, 128, 8, 2), (64, 64, 4, 4),
                                          (128, 128, 32, 8), (512, 128, 4, 1), (512, 64, 8, 2)])
def test_prefill_head_dims(dk, dv, hq, hkv):
    w = synth.custom(f"pdims{dk}x{dv}", kv_lens=[90, 200], qo_lens=[90, 37], num_qo_heads=hq,
                     num_kv_heads=hkv, head_dim_qk=dk, head_dim_vo=dv, causal=True, seed=dk)
    _run_case(w, chunk=-1)


@pytest.mark.parametrize("layout,page_size", [("NHD", 16), ("HND", 4), ("HND", 32), ("HND", 8),
                                              ("NHD", 2), ("NHD", 1)])
def test_prefill_layouts_and_pages(layout, page_size):
    """Every page size takes the cooperative kernel; below 16 tokens its copy lanes form
    their own addresses from the page-table entries streamed beside the copies."""
    w = synth.custom("playout", kv_lens=[60, 150], qo_lens=[20, 50], num_qo_heads=8,
                     num_kv_heads=2, page_size=page_size, causal=True, seed=22)
    _run_case(w, layout=layout, chunk=-1)
    if page_size < 16:
        _run_case(w, layout=layout, chunk=32)  # split items: chunks starting mid-request


@pytest.mark.parametrize("dk,dv", [(512, 256), (256, 128)])
@pytest.mark.parametrize("hkv", [2, 8])
@pytest.mark.parametrize("page_size", [1, 16])
def test_prefill_asymmetric_support_matrix(dk, dv, hkv, page_size):
    """Asymmetric prefill over (512, 256) and (256, 128), page sizes 1 and 16, two and
    eight kv heads ([PF] commit on unequal K/V strides, support half: the matrix its
    tests cover).  Ragged causal extend, two qo heads per kv head."""
    w = synth.custom(f"pasym{dk}x{dv}h{hkv}p{page_size}", kv_lens=[70, 161, 33],
                     qo_lens=[70, 40, 9], num_qo_heads=2 * hkv, num_kv_heads=hkv,
                     head_dim_qk=dk, head_dim_vo=dv, page_size=page_size, causal=True,
                     seed=dk + hkv + page_size)
    _run_case(w, chunk=-1)
    _run_case(w, chunk=32)


def test_prefill_unequal_strides():
    w = synth.custom("pstrides", kv_lens=[64, 180], qo_lens=[64, 30], num_qo_heads=8,
                     num_kv_heads=2, causal=True, seed=23)
    _run_case(w, k_pad=(1, 1, 3, 16), v_pad=(2, 0, 1, 32), chunk=-1)


@pytest.mark.parametrize("dk,dv", [(128, 128), (256, 256), (64, 64), (512, 256)])
def test_prefill_extreme_q_magnitudes(dk, dv):
    """Query rows scaled by 2^18 (|q sm_scale log2 e| far above fp16's range: those waves
    take the exactly prescaled Q) next to rows scaled by 2^-20 (fp16 subnormals once
    multiplied by the score factor) and ordinary rows.  Powers of two keep Q exact in
    bf16, so the oracle sees the same values."""
    w = synth.custom(f"pqmag{dk}", kv_lens=[150, 230], qo_lens=[70, 100], num_qo_heads=8,
                     num_kv_heads=2, head_dim_qk=dk, head_dim_vo=dv, causal=True, seed=41)
    c = gh.build_oracle_case(w)
    scale = np.ones(c.q_np.shape[0])
    scale[:12] = 2.0 ** 18          # request 0, first queries: one wave's rows and more
    scale[70:80] = 2.0 ** -20       # request 1, first queries
    c.q_np = c.q_np * scale[:, None, None]
    c.q = (c.q.double() * torch.from_numpy(scale).to(c.q.device)[:, None, None]).to(torch.bfloat16)
    assert np.array_equal(c.q.cpu().double().numpy(), c.q_np)
    plan = gh.make_plan(w, -1)
    o, lse = gh.run_gpu(c, plan)
    o_ref, lse_ref = gh.oracle_reference(c)
    gh.assert_attention_close(o, lse, o_ref, lse_ref, w.name)


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


@pytest.mark.parametrize("d,n,heads", [(64, 9, 3), (256, 13, 2), (512, 70, 1), (4, 1, 5)])
def test_merge_states_dims_and_many_parts(d, n, heads):
    """Head dims 64..512 and more parts than any fixed unroll (up to 70), with -inf
    parts, fully empty rows and one part dominating by a wide margin."""
    rng = np.random.default_rng(d + n)
    rows = 23
    o_parts = rng.standard_normal((rows, n, heads, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((rows, n, heads)) * 4).astype(np.float32)
    lse_parts[0, : max(1, n - 1)] = -np.inf        # one live part (or none when n == 1)
    lse_parts[1] = -np.inf                          # empty row
    lse_parts[2, 0] = 80.0                          # dominates the rest
    o, lse = nv.merge_states(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = ref.merge_states(np.moveaxis(o_parts, 1, 0), np.moveaxis(lse_parts, 1, 0))
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.array_equal(np.isinf(lse), np.isinf(lse_ref))
    fin = np.isfinite(lse_ref)
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= 1e-5 * max(1.0, np.abs(lse_ref[fin]).max())
    assert np.abs(o - o_ref).max() < 1e-5
    assert np.all(o[1] == 0)


def test_decode_more_than_64_partials():
    """16-token chunks over long rows: up to 71 partial states per row group, past the
    merge kernel's 8-part fast path and its 64-LSE batches."""
    w = synth.custom("manyparts", kv_lens=[4500, 1100, 16], num_qo_heads=8, num_kv_heads=2,
                     seed=61)
    _, plan = _run_case(w, chunk=16)
    assert plan.info()["num_partials"] > 64


# ------------------------------------------------------------ bad page entries --

def _new_rows(w, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    kn = torch.randn((w.batch, w.num_kv_heads, w.head_dim_qk), generator=g).to(torch.bfloat16)
    vn = torch.randn((w.batch, w.num_kv_heads, w.head_dim_vo), generator=g).to(torch.bfloat16)
    return kn, vn


@pytest.mark.parametrize("kind,page_size,chunk", [
    ("decode", 16, -1), ("decode", 16, 64), ("decode", 4, 32), ("append", 16, 64),
    ("append", 16, -1), ("prefill", 16, -1), ("prefill", 16, 64), ("prefill", 1, -1)])
@pytest.mark.parametrize("entry", ["num_pages", "minus_one"])
def test_bad_page_entry_gives_nan_rows(kind, page_size, chunk, entry):
    """A page-table entry outside [0, num_pages) is read as nothing: the rows of its
    request come out NaN (O and LSE), every other request's rows equal the oracle, and
    (append) nothing is written through it.  The kernels clamp the entry before forming
    any address, so no pool byte outside the pools is touched."""
    decode = kind != "prefill"
    lens = [150, 300, 77]
    w = synth.custom(f"badpage_{kind}", kv_lens=lens, qo_lens=None if decode else [30, 45, 20],
                     num_qo_heads=8, num_kv_heads=2, page_size=page_size, causal=False, seed=71)
    c = gh.build_oracle_case(w)
    bad = c.k_pool.num_pages if entry == "num_pages" else -1
    # request 1: its second page, or (append) the page its new token goes to
    idx = (lens[1] - 1) // page_size if kind == "append" else 1
    c.page_table[1, idx] = bad
    plan = gh.make_plan(w, chunk)
    ws = plan.new_workspace()
    plan.upload(ws)
    rows = c.q.shape[0]
    o = torch.full((rows, w.num_qo_heads, w.head_dim_vo), 7.0, device="cuda")
    lse = torch.full((rows, w.num_qo_heads), 7.0, device="cuda")
    if kind == "append":
        kn, vn = _new_rows(w, 72)
        before = (c.k_pool.data.clone(), c.v_pool.data.clone(), c.k_pool.sf.clone(),
                  c.v_pool.sf.clone())
        nv.batch_decode_append(plan, c.q, kn.cuda(), vn.cuda(), c.page_table, c.k_pool,
                               c.v_pool, w.sm_scale, ws, out=o, lse=lse)
        # the oracle's pools get the other requests' new tokens
        pt, P = c.pt, w.page_size
        for b in (0, 2):
            t = lens[b] - 1
            pg, off = pt[b, t // P], t % P
            for (data, sf), x in ((c.k_np, kn), (c.v_np, vn)):
                pk, ps = ref.quantize(x[b].double().numpy())
                data[pg, :, off], sf[pg, :, off] = pk, ps
    elif decode:
        nv.batch_decode(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o,
                        lse=lse)
    else:
        nv.batch_prefill(plan, c.q, c.page_table, c.k_pool, c.v_pool, w.sm_scale, ws, out=o,
                         lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    ind = synth.indptr(w.qo_lens)
    r0, r1 = int(ind[1]), int(ind[2])
    assert np.isnan(o[r0:r1]).all() and np.isnan(lse[r0:r1]).all()
    o_ref, lse_ref = gh.oracle_reference(c, rows=[0, 2])
    keep = np.ones(rows, dtype=bool)
    keep[r0:r1] = False
    gh.assert_attention_close(o[keep], lse[keep], o_ref[keep], lse_ref[keep], w.name)
    if kind == "append":
        # request 1's new token had no valid page: the pools hold the other two tokens'
        # new bytes and nothing else changed
        after = (c.k_pool.data, c.v_pool.data, c.k_pool.sf, c.v_pool.sf)
        changed = [torch.nonzero((a != b_).reshape(a.shape[0], -1).any(1)).flatten().tolist()
                   for a, b_ in zip(after, before)]
        allowed = {int(c.pt[b, (lens[b] - 1) // w.page_size]) for b in (0, 2)}
        for ch in changed:
            assert set(ch) <= allowed, (ch, allowed)


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


# ------------------------------------------------------------ decode + append ----

def _clone_view(t):
    base = t._base if t._base is not None else t
    nb = base.clone()
    return nb.as_strided(t.size(), t.stride(), t.storage_offset())


def _clone_pool(p):
    return nv.KVPool(_clone_view(p.data), _clone_view(p.sf), head_dim=p.head_dim,
                     layout=p.layout, global_scale=p.global_scale)


def _slot_rows(pool, page, off):
    """(data, sf) rows of one slot for every kv head."""
    if pool.layout == "HND":
        return pool.data[page, :, off], pool.sf[page, :, off]
    return pool.data[page, off], pool.sf[page, off]


@pytest.mark.gpu
@pytest.mark.parametrize("lens,hq,hkv,dk,dv,page,chunk,layout,gs,defer", [
    ([1, 32, 33, 100, 517], 8, 2, 128, 128, 16, None, "HND", (1.0, 1.0), False),
    ([1, 32, 33, 100, 517], 8, 2, 128, 128, 16, 32, "HND", (1.0, 1.0), False),
    ([0, 64, 65, 300], 4, 1, 128, 128, 16, 64, "NHD", (0.75, 1.25), True),
    ([200, 31], 32, 1, 128, 128, 16, None, "HND", (1.0, 1.0), False),
    ([97, 1000], 8, 2, 64, 64, 32, 64, "HND", (1.0, 1.0), False),
    ([129, 700], 8, 1, 512, 256, 16, 128, "HND", (1.0, 1.0), False),
    ([40, 1025], 8, 2, 256, 128, 64, None, "NHD", (1.0, 1.0), False),
])
def test_decode_append_matches_quantize_then_decode(lens, hq, hkv, dk, dv, page, chunk, layout,
                                                    gs, defer):
    """The fused append writes the oracle quantiser's bytes to the slot of every request's
    last key, and its outputs equal, bit for bit, quantize_kv into those slots followed by
    batch_decode; both match the oracle."""
    w = synth.custom("append", kv_lens=lens, num_qo_heads=hq, num_kv_heads=hkv, head_dim_qk=dk,
                     head_dim_vo=dv, page_size=page, seed=41)
    c = gh.build_oracle_case(w, layout=layout, k_global=gs[0], v_global=gs[1])
    _, k, v = synth.draw_qkv(w, device="cpu")
    last = np.cumsum(w.kv_lens) - 1
    have = np.array(w.kv_lens) > 0
    slots = synth.token_slots(w, c.pt)
    # the new rows of every request ([batch, Hkv, D]; zero rows where nothing is appended)
    k_new = torch.zeros((w.batch, hkv, dk), dtype=torch.bfloat16)
    v_new = torch.zeros((w.batch, hkv, dv), dtype=torch.bfloat16)
    k_new[have] = k[last[have]]
    v_new[have] = v[last[have]]
    k_new, v_new = k_new.cuda(), v_new.cuda()
    # poison the slots the appends will write
    rng = np.random.default_rng(5)
    for b in np.nonzero(have)[0]:
        s = int(slots[last[b]])
        for pool in (c.k_pool, c.v_pool):
            d, f = _slot_rows(pool, s // page, s % page)
            d.copy_(torch.from_numpy(rng.integers(0, 256, tuple(d.shape), dtype=np.uint8)))
            f.fill_(synth.SF_POISON)
    plan = gh.make_plan(w, chunk)
    plan.set_deferred_merge(defer)
    outs = []
    pools = []
    for fused in (False, True):
        kp, vp = _clone_pool(c.k_pool), _clone_pool(c.v_pool)
        ws = plan.new_workspace()
        plan.upload(ws)
        o = torch.full((w.batch, hq, dv), float("nan"), device="cuda")
        lse = torch.full((w.batch, hq), float("nan"), device="cuda")
        if fused:
            nv.batch_decode_append(plan, c.q, k_new, v_new, c.page_table, kp, vp, w.sm_scale, ws,
                                   out=o, lse=lse)
        else:
            sl = torch.from_numpy(np.where(have, slots[np.maximum(last, 0)], -1)).cuda()
            nv.quantize_kv(k_new, v_new, sl, kp, vp)
            nv.batch_decode(plan, c.q, c.page_table, kp, vp, w.sm_scale, ws, out=o, lse=lse)
        if defer:
            nv.merge_partials(plan, ws, o, lse)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), lse.cpu().numpy()))
        pools.append((kp, vp))
    (oa, la), (ob, lb) = outs
    assert np.array_equal(oa, ob, equal_nan=True) and np.array_equal(la, lb, equal_nan=True)
    for pa, pb, ref_pool in ((pools[0][0], pools[1][0], "k"), (pools[0][1], pools[1][1], "v")):
        assert torch.equal(pa.data, pb.data) and torch.equal(pa.sf, pb.sf), ref_pool
    # the appended slots hold the oracle quantiser's bytes (the case was built from them)
    kd, ksf = c.k_np
    vd, vsf = c.v_np
    for b in np.nonzero(have)[0]:
        s = int(slots[last[b]])
        for pool, (dref, sref) in ((pools[1][0], (kd, ksf)), (pools[1][1], (vd, vsf))):
            d, f = _slot_rows(pool, s // page, s % page)
            if layout == "HND":
                dr, fr = dref[s // page, :, s % page], sref[s // page, :, s % page]
            else:
                dr, fr = dref[s // page, s % page], sref[s // page, s % page]
            assert np.array_equal(d.cpu().numpy(), dr) and np.array_equal(f.cpu().numpy(), fr)
    o_ref, lse_ref = gh.oracle_reference(c)
    gh.assert_attention_close(ob.astype(np.float64), lb.astype(np.float64), o_ref, lse_ref,
                              "decode_append")


@pytest.mark.gpu
def test_timing_events_bracket_the_kernel():
    """Launches made while timing events are set carry them; the elapsed time is positive
    and within the host's wall time of the call; the outputs are unchanged."""
    import ctypes
    import time
    hip = ctypes.CDLL("libamdhip64.so")
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        w = synth.custom("timing", kv_lens=[700, 64, 3000], num_qo_heads=8, num_kv_heads=2, seed=16)
        c = gh.build_oracle_case(w)
        plan = gh.make_plan(w)
        o0, l0 = gh.run_gpu(c, plan)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        nv.check(nv.lib.nvfp4_set_timing_events(ev[0], ev[1]))
        try:
            o1, l1 = gh.run_gpu(c, plan)
        finally:
            nv.check(nv.lib.nvfp4_set_timing_events(None, None))
        wall_ms = (time.perf_counter() - t0) * 1e3
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value <= wall_ms
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    finally:
        for e in ev:
            hip.hipEventDestroy(e)


# ------------------------------------------------------------ KV checksum ------

def _host_checksum(c, b, h):
    """XOR of every 32-bit word of request b's K/V rows and scale rows of kv head h,
    each row taken on its own, gathered through the page table on the host."""
    w = c.w
    x = np.uint32(0)
    for arr in (c.k_np[0], c.k_np[1], c.v_np[0], c.v_np[1]):
        if arr is None:          # FP8 pools have no scale rows
            continue
        rows = ref.gather_pages(arr, c.pt[b], w.kv_lens[b], w.page_size, c.layout)[:, h]
        words = np.ascontiguousarray(rows).view(np.uint32)
        if words.size:
            x ^= np.bitwise_xor.reduce(words.ravel())
    return int(x)


@pytest.mark.parametrize("dk,dv,hq,hkv,layout,chunk,pads", [
    (128, 128, 8, 2, "HND", -1, False), (128, 128, 8, 2, "HND", 32, False),
    (64, 64, 4, 1, "NHD", 64, False), (512, 256, 8, 1, "HND", 0, False),
    (256, 128, 40, 2, "HND", 16, True), (128, 64, 4, 2, "NHD", -1, True),
    (128, 128, 32, 8, "NHD", 16, False)])
def test_kv_checksum_is_exact(dk, dv, hq, hkv, layout, chunk, pads):
    """The streaming checksum equals the XOR of the same rows' words taken on the host,
    bit for bit: every byte the decode pattern streams arrives, each exactly once, and
    nothing past a request's last key is folded in (pool slots there hold random bytes).
    Group 40 runs three blocks of qo heads over the same keys; only one streams."""
    w = synth.custom(f"cks{dk}x{dv}", kv_lens=[150, 300, 77, 0, 33, 1], num_qo_heads=hq,
                     num_kv_heads=hkv, head_dim_qk=dk, head_dim_vo=dv, seed=dk + hq)
    kw = dict(k_pad=(1, 1, 3, 16), v_pad=(2, 0, 1, 32)) if pads else {}
    c = gh.build_oracle_case(w, layout=layout, **kw)
    plan = gh.make_plan(w, chunk)
    ws = plan.new_workspace()
    plan.upload(ws)
    out = torch.full((w.batch, hkv), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    nv.kv_checksum(plan, c.page_table, c.k_pool, c.v_pool, ws, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    for b in range(w.batch):
        for h in range(hkv):
            assert int(got[b, h]) == _host_checksum(c, b, h), (b, h)
    assert got[3].tolist() == [0] * hkv
