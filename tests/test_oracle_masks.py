"""Pins of the oracle's packed custom masks against things other than themselves:
numpy's own bit packing (a library routine, little-endian bit order), the causal and
full-attention special cases, pure-Python loops on tiny shapes, and a bidirectional
multimodal-prefix mask written out by hand.  Planted mistakes check the pins bite."""
import numpy as np
import pytest

from oracle import nvfp4_ref as ref
from tests import test_oracle_attention as ta

RNG = np.random.default_rng(77)


def _random_masks(qo, kv, density=0.6):
    return [RNG.random((q, l)) < density for q, l in zip(qo, kv)]


def test_packing_matches_numpy_packbits_per_segment():
    qo, kv = [3, 1, 7, 0, 5], [11, 9, 64, 4, 13]
    masks = _random_masks(qo, kv)
    packed = ref.pack_masks(masks)
    want = np.concatenate([np.packbits(m.ravel(), bitorder="little") for m in masks])
    assert np.array_equal(packed, want)
    off, total = ref.mask_segments(qo, kv)
    assert total == packed.size
    for b, m in enumerate(masks):
        got = ref.unpack_mask_segment(packed, off[b], qo[b], kv[b])
        assert np.array_equal(got, m)
        lib = np.unpackbits(packed[off[b]:off[b] + -(-m.size // 8)], bitorder="little")
        assert np.array_equal(got.ravel(), lib[:m.size].astype(bool))


def _setup(qo, kv, hq=4, hkv=2, d=32, seed=5):
    rng = np.random.default_rng(seed)
    total = sum(kv)
    k = rng.standard_normal((total, hkv, d))
    v = rng.standard_normal((total, hkv, d))
    kd, ks = ref.quantize(k)
    vd, vs = ref.quantize(v)
    kv_ind = np.concatenate([[0], np.cumsum(kv)])
    qo_ind = np.concatenate([[0], np.cumsum(qo)])
    q = rng.standard_normal((int(qo_ind[-1]), hq, d))
    return q, kd, ks, vd, vs, kv_ind, qo_ind


def _paged(q, kd, ks, vd, vs, kv_ind, qo_ind, kv, causal, mask=None):
    """The rows in a paged pool of page size 1 (page j of request b = row kv_ind[b] + j)."""
    pt = np.zeros((len(kv), max(kv)), dtype=np.int64)
    for b, l in enumerate(kv):
        pt[b, :l] = kv_ind[b] + np.arange(l)
    pool = lambda a: a[:, :, None, :]
    return ref.paged_attention(q, pool(kd), pool(ks), pool(vd), pool(vs), pt, kv, qo_ind, 1, 0.3,
                               causal, custom_mask=mask)


def test_causal_pattern_mask_equals_causal_and_ones_equal_full():
    qo, kv = [5, 1, 9], [12, 7, 9]
    q, kd, ks, vd, vs, kv_ind, qo_ind = _setup(qo, kv)
    causal = [np.arange(l)[None, :] <= np.arange(n)[:, None] + (l - n) for n, l in zip(qo, kv)]
    a = _paged(q, kd, ks, vd, vs, kv_ind, qo_ind, kv, True)
    b = _paged(q, kd, ks, vd, vs, kv_ind, qo_ind, kv, False, ref.pack_masks(causal))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ones = [np.ones((n, l), dtype=bool) for n, l in zip(qo, kv)]
    a = _paged(q, kd, ks, vd, vs, kv_ind, qo_ind, kv, False)
    b = _paged(q, kd, ks, vd, vs, kv_ind, qo_ind, kv, True, ref.pack_masks(ones))  # mask wins
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_masked_attention_matches_naive_loops():
    qo, kv = [4, 6], [9, 13]
    q, kd, ks, vd, vs, kv_ind, qo_ind = _setup(qo, kv, seed=8)
    masks = _random_masks(qo, kv, 0.5)
    masks[1][2] = False                       # a row that sees nothing: O = 0, LSE = -inf
    o, lse = _paged(q, kd, ks, vd, vs, kv_ind, qo_ind, kv, False, ref.pack_masks(masks))
    k, v = ref.dequantize(kd, ks), ref.dequantize(vd, vs)
    for b in range(2):
        q0, q1, a0, a1 = qo_ind[b], qo_ind[b + 1], kv_ind[b], kv_ind[b + 1]
        for i in range(q1 - q0):
            vis = masks[b][i]
            if not vis.any():
                assert np.all(o[q0 + i] == 0) and np.all(np.isneginf(lse[q0 + i]))
                continue
            o_n, l_n = ta.naive_attention(q[q0 + i:q0 + i + 1], k[a0:a1][vis], v[a0:a1][vis],
                                          0.3, False)
            assert np.allclose(o[q0 + i], o_n[0], atol=1e-12)
            assert np.allclose(lse[q0 + i], l_n[0], atol=1e-12)


def test_bidirectional_multimodal_prefix():
    """A prefix of image tokens attended bidirectionally, text after it causal: the rows
    of the prefix see the whole prefix (also keys after them), the text rows everything
    up to themselves.  Written out by hand from that description."""
    n = 10
    img = 4
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            m[i, j] = (i < img and j < img) or j <= i
    qo, kv = [n], [n]
    q, kd, ks, vd, vs, kv_ind, qo_ind = _setup(qo, kv, seed=9)
    o, lse = _paged(q, kd, ks, vd, vs, kv_ind, qo_ind, kv, True, ref.pack_masks([m]))
    k, v = ref.dequantize(kd, ks), ref.dequantize(vd, vs)
    o0, _ = ta.naive_attention(q[0:1], k[:img], v[:img], 0.3, False)   # row 0 sees 4 keys
    assert np.allclose(o[0], o0[0], atol=1e-12)
    o7, _ = ta.naive_attention(q[7:8], k[:8], v[:8], 0.3, False)       # row 7: keys 0..7
    assert np.allclose(o[7], o7[0], atol=1e-12)


# ------------------------------------------------------------ planted mistakes --

def _pack_big_endian(masks):
    return np.concatenate([np.packbits(np.asarray(m, bool).ravel(), bitorder="big")
                           for m in masks])


_orig_unpack = ref.unpack_mask_segment


def _unpack_transposed(packed, byte_offset, q, L):
    return _orig_unpack(packed, byte_offset, L, q).T if q * L else _orig_unpack(packed, byte_offset, q, L)


@pytest.mark.parametrize("attr,fn", [("pack_masks", _pack_big_endian),
                                     ("unpack_mask_segment", _unpack_transposed)])
def test_planted_mistakes_fail_a_pin(attr, fn, monkeypatch):
    monkeypatch.setattr(ref, attr, fn)
    failures = 0
    for pin in (test_packing_matches_numpy_packbits_per_segment,
                test_causal_pattern_mask_equals_causal_and_ones_equal_full,
                test_masked_attention_matches_naive_loops):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, attr
