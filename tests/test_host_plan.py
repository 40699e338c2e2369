"""Planner invariants (host only): chunks tile every row group's key range with
16-aligned boundaries, partial slots and merges are consistent, and work is ordered
longest first."""
import collections

import numpy as np
import pytest

import attention_bit_paged_amd as nv
from oracle import nvfp4_ref as ref

W = {name: i for i, name in enumerate(nv._lib.WORK_FIELDS)}


def check_plan(plan, kv_lens, group, qo_lens=None, causal=False):
    work = plan.work()
    info = plan.info()
    assert len(work) == info["num_work_items"]
    lens = work[:, W["kv_end"]] - work[:, W["kv_begin"]]
    assert np.all(np.diff(lens) <= 0), "work is not ordered longest first"
    by_group = collections.defaultdict(list)
    for w in work:
        by_group[(w[W["request"]], w[W["kv_head"]], w[W["row_begin"]])].append(w)
    slots = work[:, W["partial_slot"]]
    used = slots[slots >= 0]
    assert len(np.unique(used)) == len(used) == info["num_partials"]
    assert set(used.tolist()) == set(range(info["num_partials"]))
    nmerge = 0
    for key, items in by_group.items():
        b = key[0]
        items = sorted(items, key=lambda w: w[W["kv_begin"]])
        if qo_lens is None:
            end = kv_lens[b]
        else:
            L, q = kv_lens[b], qo_lens[b]
            q0, qn = key[2], items[0][W["row_count"]]
            end = min(L, q0 + qn + L - q) if causal else L
        ref.check_chunks(end, [(w[W["kv_begin"]], w[W["kv_end"]]) for w in items])
        if len(items) == 1:
            assert items[0][W["partial_slot"]] == -1 and items[0][W["merge_index"]] == -1
        else:
            nmerge += 1
            assert all(w[W["partial_slot"]] >= 0 for w in items)
            assert len({w[W["merge_index"]] for w in items}) == 1
            if plan.info()["kv_chunk_tokens"]:
                # a decode item is one workgroup of four waves, one chunk per wave
                c = plan.info()["kv_chunk_tokens"] * (1 if info["is_prefill"] else 4)
                assert all(w[W["kv_end"]] - w[W["kv_begin"]] <= c for w in items)
    assert nmerge == info["num_merges"]
    return by_group


@pytest.mark.parametrize("chunk", [0, -1, 16, 48, 256])
def test_decode_plan_tiles_every_row(chunk):
    rng = np.random.default_rng(chunk + 100)
    kv = rng.integers(0, 3000, size=37).tolist() + [0, 1, 15, 16, 17]
    plan = nv.Plan(kv, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, kv_chunk_tokens=chunk,
                   num_cus=256)
    groups = check_plan(plan, kv, 4)
    assert len(groups) == len(kv) * 8
    for (b, g, r0), items in groups.items():
        assert r0 == 0 and items[0][W["row_count"]] == 4
    if chunk < 0:
        assert plan.info()["num_partials"] == 0


def test_decode_plan_head_blocks_for_large_groups():
    plan = nv.Plan([100, 40], num_qo_heads=40, num_kv_heads=1, head_dim_qk=128, num_cus=256,
                   kv_chunk_tokens=-1)
    groups = check_plan(plan, [100, 40], 40)
    rows = sorted((r0, items[0][W["row_count"]]) for (b, g, r0), items in groups.items() if b == 0)
    assert rows == [(0, 16), (16, 16), (32, 8)]


def test_batch_decode_config_plan():
    from attention_bit_paged_amd import synth
    w = synth.workload("batch_decode")
    plan = nv.Plan(w.kv_lens, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128,
                   kv_chunk_tokens=256, num_cus=256)
    check_plan(plan, list(w.kv_lens), 4)
    info = plan.info()
    assert info["kv_chunk_tokens"] == 256
    assert info["num_work_items"] == sum(8 * -(-l // 1024) for l in w.kv_lens)


def test_auto_split_fills_the_device_for_long_context():
    plan = nv.Plan([131072] * 8, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, num_cus=256)
    info = plan.info()
    assert info["kv_chunk_tokens"] % 32 == 0 and info["kv_chunk_tokens"] > 0
    assert info["num_work_items"] * 4 >= 256 * 8      # four waves per decode item
    check_plan(plan, [131072] * 8, 4)
    # short batch that already fills the device is not split
    plan2 = nv.Plan([300] * 512, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128, num_cus=256)
    assert plan2.info()["num_partials"] == 0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("chunk", [0, -1, 64])
def test_prefill_plan_covers_every_query(causal, chunk):
    rng = np.random.default_rng(5)
    q = rng.integers(1, 300, size=9)
    kv = q + rng.integers(0, 900, size=9)
    ind = np.concatenate([[0], np.cumsum(q)])
    plan = nv.Plan(kv.tolist(), qo_indptr=ind.tolist(), num_qo_heads=32, num_kv_heads=8,
                   head_dim_qk=128, causal=causal, kv_chunk_tokens=chunk, num_cus=256)
    groups = check_plan(plan, kv.tolist(), 4, q.tolist(), causal)
    tq = plan.info()["rows_per_item"] // 4
    for b in range(9):
        for g in range(8):
            starts = sorted(r0 for (bb, gg, r0) in groups if bb == b and gg == g)
            assert starts == list(range(0, int(q[b]), tq))

