"""Pins of the oracle's rotary position embedding against things other than itself:
the rotary of the transformers library (its Llama rotate-half form, a library
routine, also with linear position scaling), the two-dimensional case as complex
multiplication, the invariants of a rotation (norms, dependence on the position
difference only, position 0), and the alignment of query and key positions shown
through single-key custom masks: a query that sees only the key at its own position
scores the un-rotated dot product.  Planted mistakes check that the pins bite."""
import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as ref
from tests import test_oracle_attention as ta

RNG = np.random.default_rng(404)


def _library_rope(x, positions, theta, scale):
    """x [n, H, D] rotated by transformers' Llama rotary (linear scaling when scale != 1)."""
    tr = pytest.importorskip("transformers")
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    n, h, d = x.shape
    params = {"rope_type": "default", "rope_theta": float(theta)}
    if scale != 1.0:
        params = {"rope_type": "linear", "factor": float(scale), "rope_theta": float(theta)}
    cfg = tr.LlamaConfig(hidden_size=h * d, num_attention_heads=h, head_dim=d,
                         rope_parameters=params)
    emb = LlamaRotaryEmbedding(cfg)
    t = torch.from_numpy(np.ascontiguousarray(x)).permute(1, 0, 2)[None]    # [1, H, n, D]
    cos, sin = emb(t, torch.as_tensor(np.asarray(positions), dtype=torch.int64)[None])
    rq, _ = apply_rotary_pos_emb(t, t, cos, sin)
    return rq[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("d", [64, 128, 512])
@pytest.mark.parametrize("theta,scale", [(1e4, 1.0), (5e5, 4.0)])
def test_matches_library_rotary(d, theta, scale):
    x = RNG.standard_normal((40, 2, d))
    pos = RNG.integers(0, 2048, size=40)
    got = ref.apply_rope(x, pos, theta, scale)
    want = _library_rope(x, pos, theta, scale)
    # the library forms its angles in float32: about 2048 * 2^-24 rad of error
    assert np.abs(got - want).max() < 2e-3


def test_two_dims_is_complex_multiplication():
    x = RNG.standard_normal((25, 3, 2))
    pos = np.arange(25) * 7
    for scale in (1.0, 2.5):
        got = ref.apply_rope(x, pos, 1e4, scale)
        z = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos / scale)[:, None]
        assert np.allclose(got[..., 0], z.real, atol=1e-12)
        assert np.allclose(got[..., 1], z.imag, atol=1e-12)


def test_rotation_invariants():
    d = 128
    x = RNG.standard_normal((30, 2, d))
    y = RNG.standard_normal((30, 2, d))
    m, n, s = RNG.integers(0, 5000, 30), RNG.integers(0, 5000, 30), RNG.integers(0, 90000, 30)
    rx = ref.apply_rope(x, m)
    # every pair keeps its length
    pairs = lambda a: a[..., :d // 2] ** 2 + a[..., d // 2:] ** 2
    assert np.allclose(pairs(rx), pairs(x), rtol=1e-12, atol=1e-12)
    # a score depends on the position difference only
    dot = lambda a, b: (a * b).sum(-1)
    a1 = dot(ref.apply_rope(x, m), ref.apply_rope(y, n))
    a2 = dot(ref.apply_rope(x, m + s), ref.apply_rope(y, n + s))
    assert np.allclose(a1, a2, atol=1e-8)
    # position 0 is the identity; scale divides positions
    assert np.array_equal(ref.apply_rope(x, np.zeros(30, int)), x)
    assert np.allclose(ref.apply_rope(x, 3 * m, scale=3.0), ref.apply_rope(x, m), atol=1e-9)


def _request(q_len, L, hq=4, hkv=2, dk=32, dv=32, seed=5):
    rng = np.random.default_rng(seed)
    kd, ks = ref.quantize(rng.standard_normal((L, hkv, dk)))
    vd, vs = ref.quantize(rng.standard_normal((L, hkv, dv)))
    q = rng.standard_normal((q_len, hq, dk))
    return q, kd, ks, vd, vs


def _paged(q, kd, ks, vd, vs, causal, rope, mask=None, sm_scale=0.3):
    """One request in a pool of page size 1 (page j = key j)."""
    L = kd.shape[0]
    pool = lambda a: a[:, :, None, :]
    pt = np.arange(max(L, 1))[None, :]
    packed = None if mask is None else ref.pack_masks([mask])
    return ref.paged_attention(q, pool(kd), pool(ks), pool(vd), pool(vs), pt, [L],
                               [0, q.shape[0]], 1, sm_scale, causal, custom_mask=packed,
                               rope=rope)


def test_query_and_key_positions_align():
    """Row r of 5 queries over 12 keys sits at position 7 + r.  Seeing only the key at
    its own position, its LSE is the un-rotated scaled dot product and O is that key's
    value row; seeing only the key d positions away, the dot product with the key
    rotated by d."""
    qn, L = 5, 12
    q, kd, ks, vd, vs = _request(qn, L, seed=6)
    k, v = ref.dequantize(kd, ks), ref.dequantize(vd, vs)
    for dist in (0, -3, 4):
        mask = np.zeros((qn, L), dtype=bool)
        keys = []
        for r in range(qn):
            j = 7 + r + dist
            if 0 <= j < L:
                mask[r, j] = True
                keys.append((r, j))
        o, lse = _paged(q, kd, ks, vd, vs, True, (1e4, 1.0), mask)
        for r, j in keys:
            kr = ref.apply_rope(k[j:j + 1], [dist])[0]           # [hkv, D]
            for h in range(q.shape[1]):
                g = h // 2
                assert np.isclose(lse[r, h], 0.3 * np.dot(q[r, h], kr[g]), atol=1e-12)
                assert np.allclose(o[r, h], v[j, g], atol=1e-12)


def test_asymmetric_dims_rotate_the_whole_qk_dim():
    """Dk = 512, Dv = 256: the frequencies span the 256 pairs of the QK dim (the library
    rotary at head dim 512), against pure-Python attention loops."""
    qn, L = 3, 9
    q, kd, ks, vd, vs = _request(qn, L, hq=2, hkv=1, dk=512, dv=256, seed=8)
    o, lse = _paged(q, kd, ks, vd, vs, True, (1e4, 1.0))
    k, v = ref.dequantize(kd, ks), ref.dequantize(vd, vs)
    qr = _library_rope(q, np.arange(qn) + (L - qn), 1e4, 1.0)
    kr = _library_rope(k, np.arange(L), 1e4, 1.0)
    o_n, lse_n = ta.naive_attention(qr, kr, v, 0.3, True)
    assert np.allclose(o, o_n, atol=5e-3) and np.allclose(lse, lse_n, atol=5e-3)


def test_last_row_of_a_prefill_is_the_decode():
    qn, L = 4, 20
    q, kd, ks, vd, vs = _request(qn, L, seed=9)
    o, lse = _paged(q, kd, ks, vd, vs, True, (1e4, 1.0))
    o1, lse1 = _paged(q[-1:], kd, ks, vd, vs, False, (1e4, 1.0))
    assert np.allclose(o[-1], o1[0], atol=1e-12) and np.allclose(lse[-1], lse1[0], atol=1e-12)
    # and rotating changes the result (the pin is not vacuous)
    o0, _ = _paged(q[-1:], kd, ks, vd, vs, False, None)
    assert np.abs(o0[0] - o1[0]).max() > 1e-3


def test_ragged_and_paged_agree():
    qn, L = 6, 30
    q, kd, ks, vd, vs = _request(qn, L, seed=10)
    o, lse = _paged(q, kd, ks, vd, vs, True, (2e4, 2.0))
    o2, lse2 = ref.ragged_attention(q, kd, ks, vd, vs, [0, L], [0, qn], 0.3, True,
                                    rope=(2e4, 2.0))
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


# ------------------------------------------------------------ planted mistakes --

_orig_apply = ref.apply_rope
_orig_freq = ref.rope_frequencies
_orig_qpos = ref.query_positions
_orig_rotate = ref._rotate


def _apply_sign_flipped(x, positions, theta=1e4, scale=1.0):
    return _orig_apply(x, -np.asarray(positions, dtype=np.float64), theta, scale)


def _apply_interleaved(x, positions, theta=1e4, scale=1.0):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return _orig_apply(x[..., perm], positions, theta, scale)[..., inv]


def _freq_half_table(head_dim, theta=1e4, scale=1.0):
    w = _orig_freq(head_dim, theta, scale)
    w[head_dim // 4:] = 0.0          # the upper half of the table never filled
    return w


def _freq_wrong_exponent(head_dim, theta=1e4, scale=1.0):
    return _orig_freq(head_dim // 2, theta, scale).repeat(2)[:head_dim // 2]


def _qpos_from_zero(q_len, kv_len):
    return np.arange(q_len, dtype=np.int64)


def _rotate_q_only(q, k, kv_len, rope):
    if rope is None:
        return q, k
    return ref.apply_rope(q, ref.query_positions(q.shape[0], kv_len), *rope), k


@pytest.mark.parametrize("attr,fn", [("apply_rope", _apply_sign_flipped),
                                     ("apply_rope", _apply_interleaved),
                                     ("rope_frequencies", _freq_half_table),
                                     ("rope_frequencies", _freq_wrong_exponent),
                                     ("query_positions", _qpos_from_zero),
                                     ("_rotate", _rotate_q_only)])
def test_planted_mistakes_fail_a_pin(attr, fn, monkeypatch):
    monkeypatch.setattr(ref, attr, fn)
    failures = 0
    pins = [lambda: test_matches_library_rotary(128, 1e4, 1.0),
            lambda: test_matches_library_rotary(512, 5e5, 4.0),
            test_two_dims_is_complex_multiplication,
            test_query_and_key_positions_align,
            test_asymmetric_dims_rotate_the_whole_qk_dim]
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, (attr, fn.__name__)
