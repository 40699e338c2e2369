// Merge of partial attention states by their LSE.
//
// [XQA] "Support NVFP4 KV cache decode on SM120", changelog: the split-KV
// partial tiles are combined by mergeAndSaveOutTile.  For parts c with
// (O_c, lse_c): lse = M + ln sum_c exp(lse_c - M) with M = max_c lse_c and
// O = sum_c exp(lse_c - lse) O_c; a part with lse = -inf adds nothing.
#include "attn_step.h"

namespace nvfp4 {

namespace {

// Partials of split row groups, after the attention kernel: one wave per (merge
// record, row).  A row is one qo head of the group (decode) or one (query, qo head) pair
// of a query tile (prefill); each partial holds a normalised O row and its LSE.
template <int DV>
__global__ __launch_bounds__(256) void merge_partials_kernel(AttnArgs a, int n_merges, int prefill) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * 4 + wave;
  const int rows_per_merge = a.rows_per_slot;
  if (task >= (int64_t)n_merges * rows_per_merge) return;
  const int mi = (int)(task / rows_per_merge);
  const int r = (int)(task - (int64_t)mi * rows_per_merge);
  const int32_t* rec = a.merges + (int64_t)mi * kMergeFields;
  const int b = rec[0], kvh = rec[1], row0 = rec[2], nrow = rec[3], first = rec[4], np = rec[5];
  int64_t orow;
  int head;
  if (prefill) {
    // rows are (query, head) pairs, query major
    if (r >= nrow * a.group) return;
    const int qi = r / a.group;
    head = kvh * a.group + (r - qi * a.group);
    orow = (int64_t)a.qo_indptr[b] + row0 + qi;
  } else {
    if (r >= nrow) return;
    head = kvh * a.group + row0 + r;
    orow = b;
  }
  // lane covers value dims [lane * DV/64, (lane+1) * DV/64)
  constexpr int PER = DV / 64;
  float mx = -INFINITY;
  bool any_nan = false;
  for (int p = 0; p < np; ++p) {
    const float lp = a.part_lse[(int64_t)(first + p) * a.rows_per_slot + r];
    any_nan |= lp != lp;
    mx = fmaxf(mx, lp);
  }
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  if (mx > -INFINITY) {
    for (int p = 0; p < np; ++p) {
      const int64_t prow = (int64_t)(first + p) * a.rows_per_slot + r;
      const float lp = a.part_lse[prow];
      const float w = lp > -INFINITY ? __expf(lp - mx) : 0.f;
      wsum += w;
      const float* src = a.part_o + prow * DV + lane * PER;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] += w * src[k];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float* dst = a.o + orow * a.o_s_row + (int64_t)head * a.o_s_head + lane * PER;
#pragma unroll
  for (int k = 0; k < PER; ++k) dst[k] = any_nan ? NAN : acc[k] * inv;
  if (lane == 0)
    a.lse[orow * a.num_qo_heads + head] =
        any_nan ? NAN : (wsum > 0.f ? mx + __logf(wsum) : -INFINITY);
}

// Standalone merge: o_parts [rows, np, heads, D], lse_parts [rows, np, heads].
// One wave per (row, head).
__global__ __launch_bounds__(256) void merge_states_kernel(const float* __restrict__ o_parts,
                                                           const float* __restrict__ lse_parts,
                                                           int64_t rows, int np, int heads, int dim,
                                                           float* __restrict__ o,
                                                           float* __restrict__ lse) {
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pair >= rows * heads) return;
  const int64_t row = pair / heads;
  const int h = (int)(pair - row * heads);
  float mx = -INFINITY;
  for (int p = 0; p < np; ++p) mx = fmaxf(mx, lse_parts[(row * np + p) * heads + h]);
  float wsum = 0.f;
  const int c4 = dim / 4;
  float4 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (mx > -INFINITY) {
    for (int p = 0; p < np; ++p) {
      const float l = lse_parts[(row * np + p) * heads + h];
      const float w = l > -INFINITY ? __expf(l - mx) : 0.f;
      wsum += w;
      if (w == 0.f) continue;
      const float4* src = reinterpret_cast<const float4*>(o_parts + ((row * np + p) * heads + h) * dim);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = lane + 64 * k;
        if (c < c4) {
          const float4 v = src[c];
          acc[k].x += w * v.x;
          acc[k].y += w * v.y;
          acc[k].z += w * v.z;
          acc[k].w += w * v.w;
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float4* dst = reinterpret_cast<float4*>(o + (row * heads + h) * dim);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = lane + 64 * k;
    if (c < c4) dst[c] = make_float4(acc[k].x * inv, acc[k].y * inv, acc[k].z * inv, acc[k].w * inv);
  }
  if (lane == 0) lse[row * heads + h] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_merge_partials(const AttnArgs& a, int n_merges, int dv, int prefill,
                                 hipStream_t stream) {
  if (n_merges <= 0) return hipSuccess;
  const int64_t tasks = (int64_t)n_merges * a.rows_per_slot;
  const dim3 grid((unsigned)((tasks + 3) / 4));
  switch (dv) {
    case 64: hipLaunchKernelGGL(merge_partials_kernel<64>, grid, dim3(256), 0, stream, a, n_merges, prefill); break;
    case 128: hipLaunchKernelGGL(merge_partials_kernel<128>, grid, dim3(256), 0, stream, a, n_merges, prefill); break;
    case 256: hipLaunchKernelGGL(merge_partials_kernel<256>, grid, dim3(256), 0, stream, a, n_merges, prefill); break;
    case 512: hipLaunchKernelGGL(merge_partials_kernel<512>, grid, dim3(256), 0, stream, a, n_merges, prefill); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge_states(const float* o_parts, const float* lse_parts, int64_t rows,
                               int32_t num_parts, int32_t heads, int32_t head_dim, float* o,
                               float* lse, hipStream_t stream) {
  const int64_t pairs = rows * heads;
  if (pairs == 0) return hipSuccess;
  const int64_t nb = (pairs + 3) / 4;
  hipLaunchKernelGGL(merge_states_kernel, dim3((unsigned)nb), dim3(256), 0, stream, o_parts,
                     lse_parts, rows, num_parts, heads, head_dim, o, lse);
  return hipGetLastError();
}

}  // namespace nvfp4
