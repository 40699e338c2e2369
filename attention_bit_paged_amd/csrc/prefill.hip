// Paged NVFP4 prefill / extend: causal or full attention of a tile of query rows
// against a chunk of the paged cache.
//
// [PF] "Re-enable split-KV for NVFP4 KV cache in prefill path": the paged prefill
// path with in-kernel NVFP4 dequantisation, asymmetric head dims (commit on
// (qk, vo) = (512, 256): output sized by VO), causal runs, and prefix-cache extend
// where a short query attends a long cached prefix (commit "Gate split-KV off...").
// The causal mask is aligned to the end of the keys: query row i of a request with
// q_b queries and L_b keys sees keys j <= i + L_b - q_b.
//
// A work item is one workgroup of four waves: (request b, kv head g, query tile,
// chunk [kv0, kv1)).  The tile's rows are (query, qo head of the group) pairs, query
// major, so the heads that share a kv head share every K/V byte read.  Each wave owns
// NR groups of 16 rows and streams the chunk in 32-token steps with the next step's
// bytes in flight; the dequantised K and V^T operands of a step serve all the wave's
// row groups.  A split tile's partial states are merged by a separate kernel.
#include "attn_step.h"

namespace nvfp4 {

namespace {

template <int DK>
constexpr int prefill_nr() {
  return DK >= 512 ? 1 : 2;
}

template <int DK, int DV, bool PAGE16>
__global__ __launch_bounds__(256) void prefill_kernel(AttnArgs a) {
  using S = StepShape<DK, DV>;
  constexpr int NR = prefill_nr<DK>();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4;
  const int n = lane & 15;
  const int32_t* rec = a.work + (int64_t)blockIdx.x * kWorkFields;
  const int b = rec[W_REQ], kvh = rec[W_KVH], q0 = rec[W_ROW0], qn = rec[W_ROWS];
  const int kv0 = rec[W_KV0], kv1 = rec[W_KV1], slot = rec[W_SLOT];
  const int G = a.group;
  const int R = qn * G;
  const int row_base = wave * NR * 16;
  const bool wave_has_rows = row_base < R;  // uniform; rowless waves still meet the barriers
  const int qstart = a.qo_indptr[b];
  const int qlen = a.qo_indptr[b + 1] - qstart;
  const int off = a.kv_lens[b] - qlen;

  f16x8 qf[NR][S::NS];
  float sc[NR];
  int last[NR];
  bool rv[NR];
  int64_t tokrow[NR];
  int headi[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    const int r = row_base + rg * 16 + n;
    rv[rg] = r < R;
    const int qi = r / G;
    const int gh = r - qi * G;
    const int qpos = q0 + qi;
    tokrow[rg] = (int64_t)qstart + qpos;
    headi[rg] = kvh * G + gh;
    last[rg] = a.causal ? min(kv1 - 1, qpos + off) : kv1 - 1;
    sc[rg] = a.score_scale *
             load_q_operand<DK>(a.q + tokrow[rg] * a.q_s_row + (int64_t)headi[rg] * a.q_s_head,
                                rv[rg], j, qf[rg]);
  }
  // keys this wave needs: up to the last visible key of its last valid row
  int wave_end = wave_has_rows ? kv1 : kv0;
  if (a.causal && wave_has_rows) {
    const int r_last = min(R - 1, row_base + NR * 16 - 1);
    wave_end = min(kv1, q0 + r_last / G + off + 1);
  }
  // steps that may hold a masked key: the chunk's tail and, for causal rows, any step
  // past the first visible-key limit of the wave's first row
  int mask_from = kv1 - kDecodeStep;
  if (a.causal) mask_from = min(mask_from, q0 + row_base / G + off + 1 - kDecodeStep);

  PagedView<DK, DV, PAGE16> view;
  view.init(a, b, kvh, lane);
  const int tlast = kv1 - 1;

  RowState<S::NT, false> st[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) st[rg].init();

  auto step = [&](const StepRaw<DK, DV>& r, int t0) {
    f16x8 ka[S::NS], kb[S::NS];
    k_operands<DK, DV>(r, ka, kb);
    const bool masked = t0 > mask_from;
    f16x8 p[NR];
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S::NS; ++s) {
        sa = mfma16x16x32(ka[s], qf[rg][s], sa);
        sb = mfma16x16x32(kb[s], qf[rg][s], sb);
      }
      p[rg] = masked ? st[rg].template softmax<true>(sa, sb, sc[rg], t0, j, last[rg])
                     : st[rg].template softmax<false>(sa, sb, sc[rg], t0, j, last[rg]);
    }
    f16x8 vt[S::NT];
    if (t0 + kDecodeStep > kv1)
      v_operands<DK, DV, true>(r, t0, tlast, j, vt);
    else
      v_operands<DK, DV, false>(r, t0, tlast, j, vt);
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) st[rg].pv(vt, p[rg]);
  };

  StepRaw<DK, DV> r0, r1;
  if (kv0 < wave_end) view.load(r0, kv0, tlast);
  for (int t0 = kv0; t0 < wave_end; t0 += 2 * kDecodeStep) {
    const int t1 = t0 + kDecodeStep;
    if (t1 < wave_end) view.load(r1, t1, tlast);
    step(r0, t0);
    if (t1 >= wave_end) break;
    if (t1 + kDecodeStep < wave_end) view.load(r0, t1 + kDecodeStep, tlast);
    step(r1, t1);
  }

  const bool bad = __any(view.bad != 0);
  if (slot < 0) {
    if (wave_has_rows) {
#pragma unroll
      for (int rg = 0; rg < NR; ++rg)
        st[rg].store(a.o + tokrow[rg] * a.o_s_row + (int64_t)headi[rg] * a.o_s_head,
                     a.lse + tokrow[rg] * a.num_qo_heads + headi[rg], rv[rg], bad, a.out_scale, j);
    }
    return;
  }
  if (wave_has_rows) {
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      const int r = row_base + rg * 16 + n;
      st[rg].store(a.part_o + ((int64_t)slot * a.rows_per_slot + r) * DV,
                   a.part_lse + (int64_t)slot * a.rows_per_slot + r, rv[rg], bad, a.out_scale, j);
    }
  }
}

template <int DK, int DV>
hipError_t launch_dk_dv(int page_shift, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_work);
  if (page_shift >= 4)
    hipLaunchKernelGGL((prefill_kernel<DK, DV, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<DK, DV, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(int dk, int dv) {
  const bool okk = dk == 64 || dk == 128 || dk == 256 || dk == 512;
  const bool okv = dv == 64 || dv == 128 || dv == 256 || dv == 512;
  return okk && okv && dv <= dk && !(dk == 512 && dv == 512);
}

int prefill_rows_per_item(int dk, int /*dv*/, int /*group*/) { return 64 * (dk >= 512 ? 1 : 2); }

size_t prefill_lds_bytes(int /*dk*/, int /*dv*/) { return 0; }

hipError_t launch_prefill(int dk, int dv, int page_shift, const AttnArgs& a, int /*rows*/,
                          hipStream_t stream) {
  if (a.n_work <= 0) return hipSuccess;
#define NVFP4_PREFILL_CASE(K, V) \
  if (dk == K && dv == V) return launch_dk_dv<K, V>(page_shift, a, stream);
  NVFP4_PREFILL_CASE(64, 64)
  NVFP4_PREFILL_CASE(128, 64)
  NVFP4_PREFILL_CASE(128, 128)
  NVFP4_PREFILL_CASE(256, 64)
  NVFP4_PREFILL_CASE(256, 128)
  NVFP4_PREFILL_CASE(256, 256)
  NVFP4_PREFILL_CASE(512, 64)
  NVFP4_PREFILL_CASE(512, 128)
  NVFP4_PREFILL_CASE(512, 256)
#undef NVFP4_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
