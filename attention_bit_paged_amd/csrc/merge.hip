// Merge of partial attention states by their LSE.
//
// [XQA] "Support NVFP4 KV cache decode on SM120", changelog: the split-KV
// partial tiles are combined by mergeAndSaveOutTile.  For parts c with
// (O_c, lse_c): lse = M + ln sum_c exp(lse_c - M) with M = max_c lse_c and
// O = sum_c exp(lse_c - lse) O_c; a part with lse = -inf adds nothing.
#include "internal.h"

namespace nvfp4 {

namespace {

// Partials written by the decode / prefill kernels for one split row group.
__global__ __launch_bounds__(256) void merge_partials_kernel(MergeArgs m) {
  const int32_t* rec = m.merges + (int64_t)blockIdx.x * kMergeFields;
  const int b = rec[0], kvh = rec[1], row0 = rec[2], nrows_in = rec[3];
  const int first = rec[4], np = rec[5];
  const int nrows = m.prefill ? nrows_in * m.group : nrows_in;
  const int c4 = m.head_dim / 4;
  const int total = nrows * c4;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int r = idx / c4;
    const int c = idx - r * c4;
    float mx = -INFINITY;
    for (int p = 0; p < np; ++p) mx = fmaxf(mx, m.part_lse[(int64_t)(first + p) * m.rows_per_slot + r]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
    if (mx > -INFINITY) {
      for (int p = 0; p < np; ++p) {
        const int64_t prow = (int64_t)(first + p) * m.rows_per_slot + r;
        const float l = m.part_lse[prow];
        const float w = l > -INFINITY ? __expf(l - mx) : 0.f;
        if (w > 0.f) {
          const float4 v = reinterpret_cast<const float4*>(m.part_o + prow * m.head_dim)[c];
          acc.x += w * v.x;
          acc.y += w * v.y;
          acc.z += w * v.z;
          acc.w += w * v.w;
        }
        wsum += w;
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    int64_t orow;
    int head;
    if (m.prefill) {
      const int qi = r / m.group;
      head = kvh * m.group + (r - qi * m.group);
      orow = (int64_t)m.qo_indptr[b] + row0 + qi;
    } else {
      head = kvh * m.group + row0 + r;
      orow = b;
    }
    float4* dst = reinterpret_cast<float4*>(m.o + orow * m.o_s_row + (int64_t)head * m.o_s_head);
    dst[c] = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (c == 0) m.lse[orow * m.num_qo_heads + head] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
  }
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

hipError_t launch_merge_partials(const MergeArgs& m, hipStream_t stream) {
  if (m.n_merges <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_partials_kernel, dim3(m.n_merges), dim3(256), 0, stream, m);
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
