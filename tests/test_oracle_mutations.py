"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one.  A pin that no mutation can fail would not be pinning much."""
import numpy as np
import pytest

from oracle import nvfp4_ref as ref
from tests import test_oracle_attention as ta
from tests import test_oracle_formats as tf

GOLDEN = None


def _e4m3_floor(x):
    vals = ref.e4m3_value(np.arange(127))
    x = np.asarray(x, dtype=np.float64)
    return np.clip(np.searchsorted(vals, x, side="right") - 1, 0, 126).astype(np.uint8)


def _e2m1_ties_away(r):
    r = np.asarray(r, dtype=np.float64)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    return np.searchsorted(mids, r, side="right").astype(np.uint8)


def _unpack_swapped(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed >> 4
    out[..., 1::2] = packed & 0xF
    return out


_orig_attention = ref.attention
_orig_merge = ref.merge_states


def _attention_no_scale(q, k, v, sm_scale, causal=False):
    return _orig_attention(q, k, v, 1.0, causal)


def _attention_causal_off_by_one(q, k, v, sm_scale, causal=False):
    if not causal:
        return _orig_attention(q, k, v, sm_scale, causal)
    # sees one key fewer: j < i + (L - n)
    n, L = q.shape[0], k.shape[0]
    o = np.zeros((n, q.shape[1], v.shape[-1]))
    lse = np.full((n, q.shape[1]), -np.inf)
    for i in range(n):
        hi = i + (L - n)
        if hi > 0:
            o[i:i + 1], lse[i:i + 1] = _orig_attention(q[i:i + 1], k[:hi], v[:hi], sm_scale)
    return o, lse


def _attention_log2(q, k, v, sm_scale, causal=False):
    o, lse = _orig_attention(q, k, v, sm_scale, causal)
    return o, lse / np.log(2.0)


def _attention_gqa_modulo(q, k, v, sm_scale, causal=False):
    hq, hkv = q.shape[1], k.shape[1]
    idx = np.arange(hq) % hkv
    return _orig_attention(q, k[:, idx], v[:, idx], sm_scale, causal)


def _merge_unnormalised(o_parts, lse_parts):
    o, lse = _orig_merge(o_parts, lse_parts)
    return o * len(o_parts), lse


_E2M1_CODE5_WRONG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 4.0, 6.0])

MUTATIONS = {
    "e2m1 table code 5 = 2.5": ("E2M1_MAGNITUDE", _E2M1_CODE5_WRONG),
    "scale rounds down": ("e4m3_round", _e4m3_floor),
    "element ties away from zero": ("e2m1_round", _e2m1_ties_away),
    "nibble order swapped": ("unpack_nibbles", _unpack_swapped),
    "sm_scale dropped": ("attention", _attention_no_scale),
    "causal offset off by one": ("attention", _attention_causal_off_by_one),
    "lse in log2": ("attention", _attention_log2),
    "gqa head map h % Hkv": ("attention", _attention_gqa_modulo),
    "merge not normalised": ("merge_states", _merge_unnormalised),
}


def _pins(golden_dir):
    return [
        lambda: tf.test_vones_probe_matches_page(golden_dir),
        tf.test_e2m1_values_follow_the_bit_fields,
        tf.test_e2m1_ties_to_even_and_saturation,
        tf.test_e2m1_matches_brute_force,
        tf.test_e4m3_round_matches_torch_cast,
        tf.test_quantiser_is_nearest_value_brute_force,
        tf.test_quantiser_block_axis_and_nibble_order,
        lambda: ta.test_attention_matches_naive_and_torch(3, 40, 2, 1, 64, 32, True),
        lambda: ta.test_attention_matches_naive_and_torch(5, 23, 4, 2, 32, 16, False),
        lambda: ta.test_uniform_scores_give_ln_seq_len(golden_dir),
        ta.test_causal_offset_pinned_by_uniform_lse,
        ta.test_merge_of_random_aligned_chunks_equals_unsplit,
        lambda: ta.test_paged_attention_equals_dense("HND"),
    ]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_each_planted_mistake_fails_a_pin(name, golden_dir, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ref, attr, fn)
    failures = 0
    for pin in _pins(golden_dir):
        try:
            pin()
        except AssertionError:
            failures += 1
        except Exception:          # a crash also exposes the mutation
            failures += 1
    assert failures > 0, f"no pin caught: {name}"


def test_unmutated_oracle_passes_every_pin(golden_dir):
    for pin in _pins(golden_dir):
        pin()
