"""GPU parity of prefill with in-kernel RoPE against the oracle: the cooperative
kernel at every shape family (one, two and four K entries per lane and wave, the
512-dim wide kernel), pages of 4 and 1 tokens (per-lane copy addresses), NVFP4 and FP8, causal
and full, unsplit and split, ragged KV, a base and position scale other than the
defaults, and positions up to 70000 (where a plain float product pos * w would
already miss the angle by about 1e-2 rad)."""
import numpy as np
import pytest
import torch

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import synth
from oracle import nvfp4_ref as ref
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _run(w, chunk, rope, kv_dtype="nvfp4", layout="HND"):
    c = gh.build_oracle_case(w, layout=layout, kv_dtype=kv_dtype)
    plan = nv.Plan(w.kv_lens, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                   head_dim_qk=w.head_dim_qk, head_dim_vo=w.head_dim_vo, page_size=w.page_size,
                   qo_indptr=synth.indptr(w.qo_lens).tolist(), causal=w.causal,
                   kv_chunk_tokens=chunk, num_cus=256, kv_dtype=kv_dtype, rope_theta=rope[0],
                   rope_scale=rope[1])
    o, lse = gh.run_gpu(c, plan)
    o_ref, lse_ref = ref.paged_attention(c.q_np, c.k_np[0], c.k_np[1], c.v_np[0], c.v_np[1],
                                         c.pt, w.kv_lens, synth.indptr(w.qo_lens), w.page_size,
                                         w.sm_scale, w.causal, layout, kv_dtype=kv_dtype,
                                         rope=rope)
    err = gh.assert_attention_close(o, lse, o_ref, lse_ref, w.name)
    # the rotation matters at these sizes: the unrotated result is far off
    o_plain, _ = ref.paged_attention(c.q_np, c.k_np[0], c.k_np[1], c.v_np[0], c.v_np[1], c.pt,
                                     w.kv_lens, synth.indptr(w.qo_lens), w.page_size, w.sm_scale,
                                     w.causal, layout, kv_dtype=kv_dtype)
    sel = ~np.isnan(lse_ref)
    assert np.abs(o_plain[sel] - o_ref[sel]).max() > 10 * gh.O_ATOL
    print(f"rope {w.name} {kv_dtype} chunk={chunk} rope={rope}: max |O err| {err:.2e}", flush=True)
    return err


@pytest.mark.parametrize("kv_dtype", ["nvfp4", "fp8"])
@pytest.mark.parametrize("causal,chunk", [(True, -1), (True, 64), (False, 0)])
def test_rope_prefill_extend(kv_dtype, causal, chunk):
    kv, qo = [300, 64, 1100, 17, 0], [45, 64, 200, 1, 0]
    w = synth.custom("rext", kv_lens=kv, qo_lens=qo, num_qo_heads=32, num_kv_heads=8,
                     causal=causal, seed=301)
    _run(w, chunk, (1e4, 1.0), kv_dtype)


@pytest.mark.parametrize("dk,dv,kv_dtype,page_size,hq,hkv", [
    (512, 256, "nvfp4", 16, 8, 1),    # wide kernel, four K entries per lane
    (512, 128, "nvfp4", 16, 4, 2),
    (256, 128, "nvfp4", 16, 8, 2),    # four K entries per lane
    (256, 256, "fp8", 16, 8, 1),
    (128, 64, "nvfp4", 16, 8, 8),     # 192-query tiles
    (64, 64, "fp8", 16, 16, 4),       # one K entry per wave: half the lanes idle
    (64, 64, "nvfp4", 16, 4, 4),
    (128, 128, "nvfp4", 4, 8, 2),     # pages of 4 tokens
    (512, 256, "nvfp4", 1, 8, 1),
    (256, 128, "fp8", 1, 4, 2),
])
def test_rope_head_dims_types_and_pages(dk, dv, kv_dtype, page_size, hq, hkv):
    kv, qo = [200, 90, 333], [70, 90, 3]
    w = synth.custom(f"rdims{dk}x{dv}p{page_size}", kv_lens=kv, qo_lens=qo, num_qo_heads=hq,
                     num_kv_heads=hkv, head_dim_qk=dk, head_dim_vo=dv, page_size=page_size,
                     causal=True, seed=302 + dk + page_size)
    _run(w, -1, (1e4, 1.0), kv_dtype)


def test_rope_long_positions_theta_and_scale():
    """Keys up to position 70000 and a base of 5e5 with positions stretched 4x, split
    over 8 chunks; NHD pools."""
    kv, qo = [70000, 5000], [40, 64]
    w = synth.custom("rlong", kv_lens=kv, qo_lens=qo, num_qo_heads=8, num_kv_heads=2,
                     causal=True, seed=303)
    _run(w, 9344, (5e5, 4.0), "nvfp4", layout="NHD")
    _run(w, 0, (1e4, 1.0), "nvfp4", layout="NHD")


@pytest.mark.parametrize("kv_dtype", ["nvfp4", "fp8"])
def test_rope_ragged(kv_dtype):
    from attention_bit_paged_amd import paged
    kv, qo = [300, 64, 1100, 17], [45, 64, 200, 1]
    w = synth.custom("rrag", kv_lens=kv, qo_lens=qo, num_qo_heads=16, num_kv_heads=4,
                     causal=True, seed=304)
    case = paged.build_ragged_case(w, dtype=kv_dtype, start=3)
    plan = paged.make_ragged_plan(case, num_cus=256, kv_chunk_tokens=-1, rope=(1e4, 1.0))
    ws = plan.new_workspace()
    plan.upload(ws)
    o, lse = nv.batch_prefill_ragged(plan, case.q, case.k, case.v, w.sm_scale, ws)
    torch.cuda.synchronize()
    host = lambda t: None if t is None else t.cpu().numpy()
    o_ref, lse_ref = ref.ragged_attention(case.q.double().cpu().numpy(), host(case.k.data),
                                          host(case.k.sf), host(case.v.data), host(case.v.sf),
                                          case.kv_indptr, case.qo_indptr, w.sm_scale, True,
                                          kv_dtype=kv_dtype, rope=(1e4, 1.0))
    err = gh.assert_attention_close(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref,
                                    lse_ref, f"ragged rope {kv_dtype}")
    print(f"ragged rope {kv_dtype}: max |O err| {err:.2e}", flush=True)


def test_rope_zero_frequency_pairs_are_plain():
    """scale huge: every angle is at most 2e-4 rad; the rotary result then equals the
    plain kernel's within the tolerance (and the oracle's rotary reading)."""
    kv, qo = [300, 129], [45, 129]
    w = synth.custom("rtiny", kv_lens=kv, qo_lens=qo, num_qo_heads=8, num_kv_heads=2,
                     causal=True, seed=305)
    c = gh.build_oracle_case(w)
    plan = nv.Plan(w.kv_lens, num_qo_heads=8, num_kv_heads=2, head_dim_qk=128,
                   qo_indptr=synth.indptr(w.qo_lens).tolist(), causal=True, num_cus=256,
                   rope_theta=1e4, rope_scale=2e6)
    o, lse = gh.run_gpu(c, plan)
    o_p, lse_p = gh.run_gpu(c, gh.make_plan(w))
    gh.assert_attention_close(o, lse, o_p, lse_p, "tiny angles vs plain")
