// Paged NVFP4 decode: one query per request, all qo heads of one kv head per wave.
//
// [XQA] "Support NVFP4 KV cache decode on SM120", walkthrough: packed K/V and their
// scale factors are streamed from the page table, unpacked, scaled and fed to the
// matrix units; split partials are merged afterwards.  [PF] "Re-enable split-KV for
// NVFP4 KV cache in prefill path", commit "Gate split-KV off when kv_data_type is
// NVFP4" and its follow-up: decode splits the KV range into 16-token-aligned chunks
// whose partial states are merged by LSE.  [FIX] "fix(attention): correct SM120 NVFP4
// qk_correction layout, row-sum reduction, and lse", commits 1-2: the row sum reduces
// over exactly the lanes of one row; lse is ln of the sum of exp of the scaled scores.
//
// A work item (request b, kv head g, up to 16 qo heads, chunk [kv0, kv1)) is one wave;
// four independent items share a 256-thread workgroup.  The qo heads of the group are
// the N dimension of the MFMAs (padded to 16), so the K/V bytes of the chunk are read
// once for all of them.  The next step's bytes are loaded before the current step is
// computed.
#include "attn_step.h"

namespace nvfp4 {

namespace {

template <int DK, int DV, bool PAGE16>
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a) {
  using S = StepShape<DK, DV>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * 4 + wave;
  if (item >= a.n_work) return;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4;
  const int n = lane & 15;
  const int32_t* rec = a.work + (int64_t)item * kWorkFields;
  const int b = rec[W_REQ], kvh = rec[W_KVH], h0 = rec[W_ROW0], hn = rec[W_ROWS];
  const int kv0 = rec[W_KV0], kv1 = rec[W_KV1], slot = rec[W_SLOT];
  const bool head_valid = n < hn;
  const int head = kvh * a.group + h0 + n;

  f16x8 qf[S::NS];
  const float score_c =
      a.score_scale * load_q_operand<DK>(a.q + (int64_t)b * a.q_s_row + (int64_t)head * a.q_s_head,
                                         head_valid, j, qf);

  PagedView<DK, DV, PAGE16> view;
  view.init(a, b, kvh, lane);
  const int tlast = kv1 - 1;

  RowState<S::NT> st;
  st.init();
  StepRaw<DK, DV> cur, nxt;
  if (kv0 < kv1) view.load(cur, kv0, tlast);
  for (int t0 = kv0; t0 < kv1; t0 += kDecodeStep) {
    if (t0 + kDecodeStep < kv1) view.load(nxt, t0 + kDecodeStep, tlast);
    f16x8 ka[S::NS], kb[S::NS];
    k_operands<DK, DV>(cur, ka, kb);
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S::NS; ++s) {
      sa = mfma16x16x32(ka[s], qf[s], sa);
      sb = mfma16x16x32(kb[s], qf[s], sb);
    }
    const f16x8 p = st.softmax(sa, sb, score_c, t0, j, tlast);
    f16x8 vt[S::NT];
    v_operands<DK, DV>(cur, t0, tlast, j, vt);
    st.pv(vt, p);
    cur = nxt;
  }

  const bool bad = __any(view.bad != 0);
  float* dst = slot < 0 ? a.o + (int64_t)b * a.o_s_row + (int64_t)head * a.o_s_head
                        : a.part_o + ((int64_t)slot * a.rows_per_slot + n) * DV;
  float* lse_dst = slot < 0 ? a.lse + (int64_t)b * a.num_qo_heads + head
                            : a.part_lse + (int64_t)slot * a.rows_per_slot + n;
  st.store(dst, lse_dst, head_valid, bad, a.out_scale, j);
}

template <int DK, int DV>
hipError_t launch_dk_dv(int page_shift, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((a.n_work + 3) / 4);
  if (page_shift >= 4)
    hipLaunchKernelGGL((decode_kernel<DK, DV, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<DK, DV, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int dk, int dv) {
  const bool okk = dk == 64 || dk == 128 || dk == 256 || dk == 512;
  const bool okv = dv == 64 || dv == 128 || dv == 256 || dv == 512;
  return okk && okv && dv <= dk;
}

hipError_t launch_decode(int dk, int dv, int page_shift, const AttnArgs& a, hipStream_t stream) {
  if (a.n_work <= 0) return hipSuccess;
#define NVFP4_DECODE_CASE(K, V) \
  if (dk == K && dv == V) return launch_dk_dv<K, V>(page_shift, a, stream);
  NVFP4_DECODE_CASE(64, 64)
  NVFP4_DECODE_CASE(128, 64)
  NVFP4_DECODE_CASE(128, 128)
  NVFP4_DECODE_CASE(256, 64)
  NVFP4_DECODE_CASE(256, 128)
  NVFP4_DECODE_CASE(256, 256)
  NVFP4_DECODE_CASE(512, 64)
  NVFP4_DECODE_CASE(512, 128)
  NVFP4_DECODE_CASE(512, 256)
  NVFP4_DECODE_CASE(512, 512)
#undef NVFP4_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
