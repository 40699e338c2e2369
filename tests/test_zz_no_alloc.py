"""The allocation-free decode (nvfp4_batch_decode_noalloc), called through the C ABI,
against nvfp4_batch_decode with a caller workspace on the same inputs: two calls in a
row, the second with a smaller batch (so the scratch still holds the first call's
tables and partials), each equal to the workspace path bit for bit and to the oracle
within the parity tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import attention_bit_paged_amd as nv
from attention_bit_paged_amd import synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _noalloc(plan, c, o, lse):
    w = c.w
    ks, vs = c.k_pool.struct(), c.v_pool.struct()
    stream = torch.cuda.current_stream().cuda_stream
    nv.check(nv.lib.nvfp4_batch_decode_noalloc(
        plan.handle, ctypes.c_void_p(c.q.data_ptr()), c.q.stride(0), c.q.stride(1),
        ctypes.c_void_p(c.page_table.data_ptr()), c.page_table.stride(0), ctypes.byref(ks),
        ctypes.byref(vs), ctypes.c_float(w.sm_scale), ctypes.c_void_p(o.data_ptr()), o.stride(0),
        o.stride(1), ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(stream)))


def _case(w, chunk):
    c = gh.build_oracle_case(w)
    plan = gh.make_plan(w, chunk)
    # reference: the workspace entry point
    o_ref, lse_ref = gh.run_gpu(c, plan)
    o = torch.full((w.batch, w.num_qo_heads, w.head_dim_vo), float("nan"), device="cuda")
    lse = torch.full((w.batch, w.num_qo_heads), float("nan"), device="cuda")
    _noalloc(plan, c, o, lse)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref), w.name
    oo, ll = gh.oracle_reference(c)
    err = gh.assert_attention_close(o, lse, oo, ll, w.name)
    print(f"{w.name}: noalloc == workspace path bit for bit; max |O err| vs oracle {err:.2e}",
          flush=True)
    return plan


def test_noalloc_decode_matches_workspace_decode_twice():
    big = synth.custom("noalloc_big", kv_lens=[3000, 517, 1999, 64, 4000, 1, 800, 2500],
                       num_qo_heads=32, num_kv_heads=8, seed=91)
    p1 = _case(big, 256)
    assert p1.info()["num_partials"] > 0
    small = synth.custom("noalloc_small", kv_lens=[300, 45, 129], num_qo_heads=8,
                         num_kv_heads=2, seed=92)
    p2 = _case(small, 32)
    assert p2.info()["num_partials"] > 0
    assert p2.workspace_bytes < p1.workspace_bytes
