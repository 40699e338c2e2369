// Merge of partial attention states by their LSE.
//
// [XQA] "Support NVFP4 KV cache decode on SM120", changelog: the split-KV
// partial tiles are combined by mergeAndSaveOutTile.  For parts c with
// (O_c, lse_c): lse = M + ln sum_c exp(lse_c - M) with M = max_c lse_c and
// O = sum_c exp(lse_c - lse) O_c; a part with lse = -inf adds nothing.
#include <algorithm>

#include "attn_step.h"

namespace nvfp4 {

namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Partials of split row groups, after the attention kernel: one wave per (merge
// record, row).  A row is one qo head of the group (decode) or one (query, qo head) pair
// of a query tile (prefill); each partial holds a normalised O row (fp16, without the
// global V scale, which is applied here) and its LSE.  Lane
// p reads partial p's LSE; each lane sums its DV/64 value dims over the partials.  With
// at most FAST partials every load is issued at once, before any weight is known, so
// the merge costs one memory round trip after the record; more partials are taken 64
// LSEs at a time with eight row loads in flight.
template <int DV>
__global__ __launch_bounds__(256) void merge_partials_kernel(AttnArgs a, int n_merges, int prefill) {
  constexpr int FAST = 8;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // the host keeps merges x rows below 2^31
  const int task = (int)blockIdx.x * 4 + wave;
  // rows a merge can have: a decode merge holds at most one block of qo heads
  const int rows_per_merge = prefill ? a.rows_per_slot : min(a.group, kDecodeHeads);
  if (task >= n_merges * rows_per_merge) return;
  const int mi = task / rows_per_merge;
  const int r = task - mi * rows_per_merge;
  // the whole record in one scalar load (records are 32-byte aligned)
  typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
  static_assert(kMergeFields == 8, "merge record");
  const i32x8 rec = *reinterpret_cast<const i32x8*>(a.merges + (int64_t)mi * kMergeFields);
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
  constexpr int PER = DV / 64;  // lane covers value dims [lane * PER, (lane + 1) * PER)
  const int64_t rps = a.rows_per_slot;
  const int64_t row_of_first = (int64_t)first * rps + r;  // partial p: row_of_first + p * rps
  const _Float16* src = a.part_o + row_of_first * DV + lane * PER;
  const int64_t step = rps * DV;
  auto lse_of = [&](int p) { return p < np ? a.part_lse[row_of_first + (int64_t)p * rps] : -INFINITY; };
  // PER consecutive fp16 values in one load (2, 4, 8 or 16 bytes)
  auto load_row = [&](const _Float16* s, float (&v)[PER]) {
    typedef _Float16 hv __attribute__((ext_vector_type(PER)));
    const hv x = *reinterpret_cast<const hv*>(s);
#pragma unroll
    for (int k = 0; k < PER; ++k) v[k] = (float)x[k];
  };
  auto lane_weight = [&](float w, int q) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), q));
  };

  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float mx, wsum = 0.f;
  bool any_nan;
  if (np <= FAST) {
    const float lp = lse_of(lane);
    float v[FAST][PER];
    // only the partials that exist (np is wave-uniform: scalar branches between loads
    // that are all in flight together)
#pragma unroll
    for (int q = 0; q < FAST; ++q)
      if (q < np) load_row(src + q * step, v[q]);
    any_nan = __any(lp != lp);
    mx = wave_max(lp);
    if (mx > -INFINITY) {
      const float w = lp > -INFINITY ? __expf(lp - mx) : 0.f;  // 0 on lanes >= np
      wsum = wave_sum(w);
#pragma unroll
      for (int q = 0; q < FAST; ++q) {
        if (q < np) {
          const float wq = lane_weight(w, q);
#pragma unroll
          for (int k = 0; k < PER; ++k) acc[k] += wq * v[q][k];
        }
      }
    }
  } else {
    mx = -INFINITY;
    bool nan = false;
    for (int p0 = 0; p0 < np; p0 += 64) {
      const float lp = lse_of(p0 + lane);
      nan |= lp != lp;
      mx = fmaxf(mx, lp);
    }
    mx = wave_max(mx);
    any_nan = __any(nan);
    if (mx > -INFINITY) {
      for (int p0 = 0; p0 < np; p0 += 64) {
        const float lp = lse_of(p0 + lane);
        const float w = lp > -INFINITY ? __expf(lp - mx) : 0.f;  // weight of partial p0 + lane
        wsum += w;
        const int cnt = min(64, np - p0);
        const _Float16* base = src + (int64_t)p0 * step;
        auto add = [&](int q) {
          const float wq = lane_weight(w, q);
          float v[PER];
          load_row(base + q * step, v);
#pragma unroll
          for (int k = 0; k < PER; ++k) acc[k] += wq * v[k];
        };
        int q = 0;
        for (; q + 8 <= cnt; q += 8) {
#pragma unroll
          for (int u = 0; u < 8; ++u) add(q + u);
        }
        for (; q < cnt; ++q) add(q);
      }
      wsum = wave_sum(wsum);
    }
  }
  const float inv = wsum > 0.f ? *a.part_scale / wsum : 0.f;
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
  const int64_t tasks =
      (int64_t)n_merges * (prefill ? a.rows_per_slot : std::min(a.group, kDecodeHeads));
  if (tasks + 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;  // 32-bit task index
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
