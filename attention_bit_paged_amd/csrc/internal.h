// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_attn.h"

namespace nvfp4 {

// Work-item record: eight int32 fields (see nvfp4_plan_get_work).
enum WorkField {
  W_REQ = 0,    // request index b
  W_KVH = 1,    // kv head
  W_ROW0 = 2,   // first qo head within the group (decode) / first query row of the tile (prefill)
  W_ROWS = 3,   // qo heads (decode) / query rows (prefill) covered
  W_KV0 = 4,    // first key of the chunk
  W_KV1 = 5,    // one past the last key of the chunk
  W_SLOT = 6,   // partial slot, or -1 when the item owns the whole row range
  W_MERGE = 7,  // merge entry, or -1
};
constexpr int kWorkFields = 8;

// Merge record: {req, kv_head, row0, rows, first_partial, num_parts, 0, 0}.
constexpr int kMergeFields = 8;

// Decode: one wave handles at most this many qo heads of one kv head.
constexpr int kDecodeHeads = 16;
// Tokens one decode wave consumes per step (two 16-row MFMA tiles).
constexpr int kDecodeStep = 32;

struct PoolArgs {
  const uint8_t* data;
  int64_t s_page, s_head, s_tok;
  const uint8_t* sf;
  int64_t sf_page, sf_head, sf_tok;
  int32_t num_pages;
};

struct AttnArgs {
  const uint16_t* q;        // bf16 bits
  int64_t q_s_row, q_s_head;
  const int32_t* page_table;
  int64_t pt_stride;
  PoolArgs k, v;
  float score_scale;        // sm_scale * log2(e) * global_scale(K)
  float out_scale;          // global_scale(V)
  const int32_t* work;      // device work records
  int32_t n_work;
  const int32_t* qo_indptr; // device, [batch + 1] (prefill)
  const int32_t* kv_lens;   // device, [batch]
  float* o;
  int64_t o_s_row, o_s_head;
  float* lse;               // [rows, num_qo_heads]
  // [slots, rows_per_slot, head_dim_vo] in fp16, without the global V scale (the merge
  // applies it)
  _Float16* part_o;
  float* part_lse;          // [slots, rows_per_slot]
  // one float of the workspace: the global V scale of the last attention launch, which
  // the merge applies to the partials (written by the first workgroup of every launch)
  float* part_scale;
  int32_t num_qo_heads;
  int32_t group;            // qo heads per kv head
  int32_t page_shift;       // log2(page_size)
  int32_t rows_per_slot;
  int32_t causal;
  // Decode: deal each run of 64 work items to the XCDs in groups of eight consecutive
  // items (see decode_item); set when the pools interleave kv heads at a short stride.
  int32_t xcd_group;
  // Decode: the K/V copies take the non-temporal cache policy (kStreamCopies), since
  // each byte is read by one work item; clear when the heads share cache lines
  // (xcd_group), whose other head's item reads them again.
  int32_t stream_kv;
  const int32_t* merges;    // merge records
  // Prefill with a custom mask (else null): packed bits, and each request's byte offset
  // into them (device, from the workspace).
  const uint8_t* mask;
  const int64_t* mask_off;
  // Prefill with in-kernel RoPE (else null): per pair i < Dk/2 of head-dim elements
  // (i, i + Dk/2), the float pair (hi, lo) with hi + lo = w_i / (2 pi) (device, from
  // the workspace).
  const float* rope;
  // Decode with append: the step's new K/V rows (bf16 [batch, kv heads, dim], element
  // strides), quantised into the slot of token kv_len-1 of their request by the work
  // item that ends there; k_new is null when the call appends nothing.
  const uint16_t* k_new;
  int64_t kn_s_req, kn_s_head;
  const uint16_t* v_new;
  int64_t vn_s_req, vn_s_head;
  double k_gscale, v_gscale;  // the pools' global scales (the quantiser's divisor)
};

struct QuantArgs {
  int32_t fp8;              // the pool stores FP8 e4m3 bytes (else NVFP4)
  const uint16_t* src;      // bf16 bits
  int64_t s_tok, s_head;    // elements
  uint8_t* data;
  int64_t d_page, d_head, d_tok;
  uint8_t* sf;
  int64_t sf_page, sf_head, sf_tok;
  int64_t num_slots;        // num_pages * page_size
  int32_t page_shift;
  int32_t num_heads;
  int32_t head_dim;
  double gscale;
};

// Timing events of the attention launches (nvfp4_set_timing_events): while set, the
// decode and prefill kernels are launched with them, so that the dispatch itself
// timestamps the kernel's start and end.  Per host thread.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

// Launches an attention (or streaming) kernel, with the thread's timing events when
// they are set.
template <typename K, typename... Args>
inline void launch_attention(K kernel, dim3 grid, dim3 block, hipStream_t stream,
                             const Args&... args) {
  const LaunchEvents& ev = launch_events();
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}

// Launchers (defined in the .hip files).  Return the hipGetLastError() status of the launch.
hipError_t launch_quantize(const QuantArgs* k, const QuantArgs* v, int64_t n_tokens,
                           const int64_t* slots, hipStream_t stream);
// `fmt` below: the pools' storage format, 0 = NVFP4, 1 = FP8 e4m3 (KvFmt).
hipError_t launch_decode(int dk, int dv, int fmt, int page_shift, const AttnArgs& a,
                         hipStream_t stream);
// Zeroes out[batch * num_kv_heads], then XORs in the KV words a decode plan streams.
hipError_t launch_kv_checksum(int dk, int dv, int fmt, const AttnArgs& a, uint32_t* out,
                              int batch, int num_kv_heads, hipStream_t stream);
bool decode_supported(int dk, int dv, int fmt);
// The shape has the ring kernel (pages of 16+ tokens; the checksum streams through it).
bool decode_ring_supported(int dk, int dv, int fmt);
// Decode workgroups (four waves each) one CU runs at once for this shape.
int decode_wgs_per_cu(int dk, int dv, int fmt);
// LDS one CU's resident decode workgroups use (any head dims of the set 64..512).
size_t decode_lds_bytes(int dk, int dv, int page_size, int fmt);
hipError_t launch_prefill(int dk, int dv, int fmt, int page_shift, const AttnArgs& a,
                          hipStream_t stream);
// The rotary (a.rope) instantiations of launch_prefill's kernels.
hipError_t launch_prefill_rope(int dk, int dv, int fmt, int page_shift, const AttnArgs& a,
                               hipStream_t stream);
bool prefill_supported(int dk, int dv, int fmt);
int prefill_rows_per_item(int dk, int dv, int group, int page_size);
// Prefill workgroups one CU runs at once for this shape.
int prefill_wgs_per_cu(int dk, int dv);
// LDS one CU's resident prefill workgroups use (any head dims of the set 64..512).
size_t prefill_lds_bytes(int dk, int dv, int page_size, int fmt);
hipError_t launch_merge_partials(const AttnArgs& a, int n_merges, int dv, int prefill,
                                 hipStream_t stream);
hipError_t launch_merge_states(const float* o_parts, const float* lse_parts, int64_t rows,
                               int32_t num_parts, int32_t heads, int32_t head_dim, float* o,
                               float* lse, hipStream_t stream);

}  // namespace nvfp4
