"""Pins of the oracle's FP8 e4m3 KV type and its ragged (non-paged) layout against
things other than themselves: torch's float8_e4m3fn conversions (a library RNE cast),
the saturation rule, and the equivalence of the ragged and the paged layouts holding
the same rows.  Planted mistakes at the end check that these pins bite."""
import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as ref
from tests import test_oracle_attention as ta

RNG = np.random.default_rng(2024)


def _torch_fp8(x):
    """torch's RNE cast of float32 values to e4m3fn bytes."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


# midpoints between neighbouring e4m3 values: exact ties in float32
_POS = ref.e4m3_value(np.arange(127))
_TIES = (_POS[:-1] + _POS[1:]) / 2


@pytest.mark.parametrize("g", [1.0, 0.5, 4.0])
def test_fp8_quantiser_matches_torch_cast(g):
    x = np.concatenate([
        RNG.standard_normal(200000) * 3,
        np.exp2(RNG.uniform(-12, 8.8, 100000)) * RNG.choice([-1, 1], 100000),
        RNG.uniform(-2.0 ** -6, 2.0 ** -6, 50000),        # subnormal range
        _TIES, -_TIES, [0.0, -0.0, 1e-30, -1e-30, 448.0, -448.0, 464.0],
    ]).astype(np.float32).astype(np.float64) * g
    got = ref.quantize_fp8(x, g)
    want = _torch_fp8(x / g)                              # x / g exact: g is a power of two
    assert np.array_equal(got, want)


def test_fp8_quantiser_saturates_and_keeps_the_sign_of_zero():
    x = np.array([465.0, 1e6, -500.0, -1e30, -0.0, -1e-30, 0.0])
    assert ref.quantize_fp8(x).tolist() == [0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x80, 0x00]
    assert ref.quantize_fp8(np.array([900.0]), 2.0).tolist() == [0x7E]


def test_fp8_dequantiser_matches_torch_for_every_code():
    codes = np.arange(256)
    tv = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for g in (1.0, 0.25, 3.0):
        ov = ref.dequantize_fp8(codes, g)
        assert np.array_equal(np.isnan(ov), np.isnan(tv))
        ok = ~np.isnan(tv)
        assert np.array_equal(ov[ok], tv[ok] * g)


def _ragged_and_paged(kv_dtype, lens, qo, hq, hkv, dk, dv, page, seed):
    """The same K/V rows laid out ragged (back to back) and paged (a shuffled pool)."""
    rng = np.random.default_rng(seed)
    total = sum(lens)
    k = rng.standard_normal((total, hkv, dk))
    v = rng.standard_normal((total, hkv, dv))
    if kv_dtype == "nvfp4":
        kd, ks = ref.quantize(k)
        vd, vs = ref.quantize(v)
    else:
        kd, ks = ref.quantize_fp8(k), None
        vd, vs = ref.quantize_fp8(v), None
    kv_ind = np.concatenate([[0], np.cumsum(lens)])
    qo_ind = np.concatenate([[0], np.cumsum(qo)])
    q = rng.standard_normal((int(qo_ind[-1]), hq, dk))
    pages = [-(-l // page) for l in lens]
    npool = sum(pages) + 3
    perm = rng.permutation(npool)
    pt = np.zeros((len(lens), max(pages)), dtype=np.int64)

    def pool_of(rows):
        if rows is None:
            return None
        pool = rng.integers(0, 256, (npool, hkv, page, rows.shape[-1]), dtype=np.uint8)
        pos = 0
        for b, l in enumerate(lens):
            for t in range(l):
                pool[perm[pos + t // page], :, t % page] = rows[kv_ind[b] + t]
            pos += pages[b]
        return pool

    pos = 0
    for b, n in enumerate(pages):
        pt[b, :n] = perm[pos:pos + n]
        pos += n
    paged = (pool_of(kd), pool_of(ks), pool_of(vd), pool_of(vs), pt)
    return q, (kd, ks, vd, vs), kv_ind, qo_ind, paged


@pytest.mark.parametrize("kv_dtype", ["nvfp4", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_equals_paged_on_the_same_rows(kv_dtype, causal):
    lens, qo = [37, 5, 64, 19], [10, 5, 64, 1]
    q, rows, kv_ind, qo_ind, paged = _ragged_and_paged(kv_dtype, lens, qo, 4, 2, 32, 32, 8, 3)
    o_r, l_r = ref.ragged_attention(q, *rows, kv_ind, qo_ind, 0.3, causal, kv_dtype=kv_dtype)
    kp, ksp, vp, vsp, pt = paged
    o_p, l_p = ref.paged_attention(q, kp, ksp, vp, vsp, pt, lens, qo_ind, 8, 0.3, causal,
                                   kv_dtype=kv_dtype)
    assert np.array_equal(o_r, o_p) and np.array_equal(l_r, l_p)


@pytest.mark.parametrize("kv_dtype", ["nvfp4", "fp8"])
def test_ragged_matches_naive_loops_on_tiny_shapes(kv_dtype):
    """Per request, the ragged oracle equals the pure-Python loops on the dequantised
    rows (dequantised here by torch for FP8, by the oracle's pinned NVFP4 decoder)."""
    lens, qo = [9, 17], [3, 17]
    q, (kd, ks, vd, vs), kv_ind, qo_ind, _ = _ragged_and_paged(kv_dtype, lens, qo, 2, 1, 32, 16,
                                                               4, 5)
    o, lse = ref.ragged_attention(q, kd, ks, vd, vs, kv_ind, qo_ind, 0.25, True, kv_dtype=kv_dtype)
    if kv_dtype == "fp8":
        dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        k, v = dec(kd), dec(vd)
    else:
        k, v = ref.dequantize(kd, ks), ref.dequantize(vd, vs)
    for b in range(2):
        a0, a1, q0, q1 = kv_ind[b], kv_ind[b + 1], qo_ind[b], qo_ind[b + 1]
        o_n, l_n = ta.naive_attention(q[q0:q1], k[a0:a1], v[a0:a1], 0.25, True)
        assert np.allclose(o[q0:q1], o_n, atol=1e-12) and np.allclose(lse[q0:q1], l_n, atol=1e-12)


# ------------------------------------------------------------ planted mistakes --

def _fp8_truncating(x, global_scale=1.0):
    x = np.asarray(x, dtype=np.float64)
    vals = ref.e4m3_value(np.arange(127))
    mag = np.clip(np.searchsorted(vals, np.abs(x) / global_scale, side="right") - 1, 0, 126)
    return ((np.signbit(x).astype(np.uint8) << 7) | mag.astype(np.uint8)).astype(np.uint8)


_orig_ragged = ref.ragged_attention


def _ragged_off_by_one(q, k_rows, k_sf, v_rows, v_sf, kv_indptr, qo_indptr, *a, **kw):
    shifted = np.asarray(kv_indptr).copy()
    shifted[1:-1] += 1
    return _orig_ragged(q, k_rows, k_sf, v_rows, v_sf, shifted, qo_indptr, *a, **kw)


@pytest.mark.parametrize("attr,fn", [("quantize_fp8", _fp8_truncating),
                                     ("ragged_attention", _ragged_off_by_one)])
def test_planted_mistakes_fail_a_pin(attr, fn, monkeypatch):
    monkeypatch.setattr(ref, attr, fn)
    pins = [lambda: test_fp8_quantiser_matches_torch_cast(1.0),
            lambda: test_ragged_equals_paged_on_the_same_rows("fp8", True),
            lambda: test_ragged_equals_paged_on_the_same_rows("nvfp4", False)]
    failures = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures > 0, attr
