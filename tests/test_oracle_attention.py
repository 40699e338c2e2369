"""Pins of the oracle's attention, paging and merge against closed forms, the
pages' worked values, brute force and a library attention routine."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as ref

RNG = np.random.default_rng(777)


def naive_attention(q, k, v, sm_scale, causal):
    """Pure-Python loops with math.fsum (tiny shapes only)."""
    n, hq, dk = q.shape
    L, hkv, _ = k.shape
    dv = v.shape[-1]
    grp = hq // hkv
    o = np.zeros((n, hq, dv))
    lse = np.full((n, hq), -math.inf)
    for i in range(n):
        for h in range(hq):
            g = h // grp
            js = [j for j in range(L) if (not causal or j <= i + L - n)]
            if not js:
                continue
            s = {j: sm_scale * math.fsum(q[i, h, d] * k[j, g, d] for d in range(dk)) for j in js}
            m = max(s.values())
            w = {j: math.exp(s[j] - m) for j in js}
            ell = math.fsum(w.values())
            lse[i, h] = m + math.log(ell)
            for d in range(dv):
                o[i, h, d] = math.fsum(w[j] * v[j, g, d] for j in js) / ell
    return o, lse


def torch_attention(q, k, v, sm_scale, causal):
    """torch fp64 scaled_dot_product_attention with an explicit mask, plus logsumexp."""
    n, hq, _ = q.shape
    L, hkv, _ = k.shape
    grp = hq // hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)                        # [hq, n, dk]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(grp, 0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(grp, 0)
    mask = torch.ones(n, L, dtype=torch.bool)
    if causal:
        mask = torch.arange(L)[None, :] <= (torch.arange(n)[:, None] + (L - n))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=sm_scale)
    s = (tq @ tk.transpose(1, 2)) * sm_scale
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def nvfp4_kv(L, hkv, d, scale=1.0):
    x = torch.from_numpy(RNG.standard_normal((L, hkv, d)) * scale).to(torch.bfloat16)
    packed, sf = ref.quantize(x.to(torch.float64).numpy())
    return packed, sf, ref.dequantize(packed, sf)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,L,hq,hkv,dk,dv", [(1, 17, 4, 1, 32, 32), (5, 23, 4, 2, 32, 16),
                                            (7, 7, 2, 2, 32, 32), (3, 40, 2, 1, 64, 32)])
def test_attention_matches_naive_and_torch(n, L, hq, hkv, dk, dv, causal):
    q = torch.from_numpy(RNG.standard_normal((n, hq, dk))).to(torch.bfloat16).double().numpy()
    _, _, k = nvfp4_kv(L, hkv, dk)
    _, _, v = nvfp4_kv(L, hkv, dv)
    sm = 1 / math.sqrt(dk)
    o, lse = ref.attention(q, k, v, sm, causal)
    on, ln = naive_attention(q, k, v, sm, causal)
    ot, lt = torch_attention(q, k, v, sm, causal)
    assert np.allclose(o, on, atol=1e-12, rtol=0) and np.allclose(lse, ln, atol=1e-12, rtol=0)
    assert np.allclose(o, ot, atol=1e-12, rtol=0) and np.allclose(lse, lt, atol=1e-12, rtol=0)


def test_uniform_scores_give_ln_seq_len(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "uniform_lse.json")))
    for L in g["seq_lens"]:
        _, _, k = nvfp4_kv(L, 1, 32)
        _, _, v = nvfp4_kv(L, 1, 32)
        q = np.zeros((1, 4, 32))
        o, lse = ref.attention(q, k, v, 0.125, False)
        assert np.all(np.abs(lse - math.log(L)) <= 1e-12 * max(1, math.log(L)))
        assert np.allclose(o, v.mean(axis=0)[0][None, None, :], atol=1e-12)


def test_uniform_scores_vones_gives_quantised_one(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "vones_probe.json")))
    L = 300
    _, _, k = nvfp4_kv(L, 2, 64)
    vp, vs = ref.quantize(np.ones((L, 2, 64)))
    v = ref.dequantize(vp, vs)
    o, _ = ref.attention(np.zeros((1, 8, 64)), k, v, 0.125, False)
    assert np.all(np.abs(o - 1.03125) < 1e-13)
    assert round(float(o[0, 0, 0]), g["printed_fixed_decimals"]) == g["printed_fixed"]


def test_causal_offset_pinned_by_uniform_lse():
    n, L = 9, 30
    _, _, k = nvfp4_kv(L, 1, 32)
    _, _, v = nvfp4_kv(L, 1, 32)
    o, lse = ref.attention(np.zeros((n, 2, 32)), k, v, 0.1, True)
    for i in range(n):
        assert abs(lse[i, 0] - math.log(i + 1 + L - n)) < 1e-12
        assert np.allclose(o[i, 0], v[: i + 1 + L - n, 0].mean(axis=0), atol=1e-12)


def test_single_key():
    q = RNG.standard_normal((1, 4, 32))
    _, _, k = nvfp4_kv(1, 1, 32)
    _, _, v = nvfp4_kv(1, 1, 32)
    o, lse = ref.attention(q, k, v, 0.3, False)
    assert np.allclose(o[0], np.repeat(v[0], 4, axis=0), atol=0, rtol=0)
    assert np.allclose(lse[0], 0.3 * q[0] @ k[0, 0], atol=1e-13)


def test_empty_request():
    o, lse = ref.attention(np.ones((1, 2, 32)), np.zeros((0, 1, 32)), np.zeros((0, 1, 16)), 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_causal_single_query_equals_noncausal():
    q = RNG.standard_normal((1, 4, 32))
    _, _, k = nvfp4_kv(50, 2, 32)
    _, _, v = nvfp4_kv(50, 2, 32)
    a = ref.attention(q, k, v, 0.2, True)
    b = ref.attention(q, k, v, 0.2, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_gqa_equals_mha_on_repeated_kv():
    q = RNG.standard_normal((3, 8, 32))
    _, _, k = nvfp4_kv(20, 2, 32)
    _, _, v = nvfp4_kv(20, 2, 32)
    o1, l1 = ref.attention(q, k, v, 0.2, True)
    o2, l2 = ref.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.2, True)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)
    # a plausible wrong mapping (h % Hkv) gives a different answer
    q2 = q.copy()
    q2[:, 1] += 1
    o3, _ = ref.attention(q2, k, v, 0.2, True)
    assert np.allclose(o3[:, [0, 2, 3, 4, 5, 6, 7]], o1[:, [0, 2, 3, 4, 5, 6, 7]], atol=1e-14)


def _paged_setup(lens, hkv, d, P, layout, seed):
    rng = np.random.default_rng(seed)
    counts = [-(-l // P) for l in lens]
    pool_pages = sum(counts) + 5
    perm = rng.permutation(pool_pages)
    pt = np.zeros((len(lens), max(counts)), dtype=np.int32)
    pos = 0
    for b, c in enumerate(counts):
        pt[b, :c] = perm[pos:pos + c]
        pos += c
    shape = (pool_pages, hkv, P, d // 2) if layout == "HND" else (pool_pages, P, hkv, d // 2)
    sshape = shape[:-1] + (d // 16,)
    pool = rng.integers(0, 256, shape, dtype=np.uint8)
    spool = np.full(sshape, 0x7F, dtype=np.uint8)
    logical = []
    for b, L in enumerate(lens):
        x = torch.from_numpy(rng.standard_normal((L, hkv, d))).to(torch.bfloat16).double().numpy()
        p, s = ref.quantize(x)
        for j in range(L):
            page, slot = pt[b, j // P], j % P
            if layout == "HND":
                pool[page, :, slot], spool[page, :, slot] = p[j], s[j]
            else:
                pool[page, slot], spool[page, slot] = p[j], s[j]
        logical.append(ref.dequantize(p, s))
    return pool, spool, pt, logical


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_paged_attention_equals_dense(layout):
    lens = [33, 16, 1, 47]
    P, hkv, hq, d = 16, 2, 4, 32
    kp, ks, pt, kl = _paged_setup(lens, hkv, d, P, layout, 1)
    vp, vs, _, _ = _paged_setup(lens, hkv, d, P, layout, 1)  # same pt; V = K values here
    q = RNG.standard_normal((len(lens), hq, d))
    ind = np.arange(len(lens) + 1)
    o, lse = ref.paged_attention(q, kp, ks, vp, vs, pt, lens, ind, P, 0.2, layout=layout)
    for b, L in enumerate(lens):
        od, ld = ref.attention(q[b:b + 1], kl[b], kl[b], 0.2)
        assert np.allclose(o[b], od[0], atol=1e-14) and np.allclose(lse[b], ld[0], atol=1e-14)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))   # poisoned slots never read


def test_page_permutation_invariance():
    lens = [40, 70]
    a = _paged_setup(lens, 1, 32, 16, "HND", 5)
    rng = np.random.default_rng(9)
    perm = rng.permutation(a[0].shape[0])          # physical page p moves to perm[p]
    kp2 = np.empty_like(a[0]); kp2[perm] = a[0]
    ks2 = np.empty_like(a[1]); ks2[perm] = a[1]
    pt2 = perm[a[2]].astype(np.int32)
    q = RNG.standard_normal((2, 2, 32))
    ind = np.arange(3)
    r1 = ref.paged_attention(q, a[0], a[1], a[0], a[1], a[2], lens, ind, 16, 0.3)
    r2 = ref.paged_attention(q, kp2, ks2, kp2, ks2, pt2, lens, ind, 16, 0.3)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_merge_of_random_aligned_chunks_equals_unsplit():
    L, hq = 333, 4
    q = RNG.standard_normal((1, hq, 32))
    _, _, k = nvfp4_kv(L, 1, 32)
    _, _, v = nvfp4_kv(L, 1, 32)
    o_full, l_full = ref.attention(q, k, v, 0.2)
    for trial in range(5):
        cuts = sorted(set(RNG.choice(np.arange(16, L, 16), size=RNG.integers(1, 8), replace=False)))
        bounds = [0] + list(cuts) + [L]
        chunks = list(zip(bounds[:-1], bounds[1:]))
        ref.check_chunks(L, chunks)
        parts = [ref.attention(q, k[a:b], v[a:b], 0.2) for a, b in chunks]
        o, lse = ref.merge_states([p[0] for p in parts], [p[1] for p in parts])
        assert np.allclose(o, o_full, atol=1e-13) and np.allclose(lse, l_full, atol=1e-13)


def test_merge_identity_and_empty_parts():
    o1 = RNG.standard_normal((1, 3, 8))
    l1 = RNG.standard_normal((1, 3))
    o, l = ref.merge_states(o1, l1)
    assert np.allclose(o, o1[0]) and np.allclose(l, l1[0])
    o, l = ref.merge_states(np.stack([o1[0], np.full((3, 8), 7.0)]),
                            np.stack([l1[0], np.full(3, -np.inf)]))
    assert np.allclose(o, o1[0]) and np.allclose(l, l1[0])
    o, l = ref.merge_states(np.zeros((2, 3, 8)), np.full((2, 3), -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_check_chunks_rejects_bad_tilings():
    ref.check_chunks(100, [(0, 32), (32, 100)])
    ref.check_chunks(0, [(0, 0)])
    for bad in ([(0, 30), (30, 100)], [(0, 32), (48, 100)], [(0, 32), (32, 32), (32, 100)],
                [(0, 96)], [(16, 100)]):
        with pytest.raises(AssertionError):
            ref.check_chunks(100, bad)
