// Host side of the C ABI: argument validation, the split-KV planner, workspace
// layout and kernel launches.  No device memory is allocated here.
//
// [PF] "Re-enable split-KV for NVFP4 KV cache in prefill path":
//   * commit "Re-enable split-KV...": reject a tile that does not fit on-chip memory
//     at plan time instead of failing at launch;
//   * commit "Gate split-KV off when kv_data_type is NVFP4", follow-up: the split of
//     the KV range uses 16-token-aligned chunk boundaries;
//   * commits on unequal K/V strides: either support them or reject them loudly
//     (supported everywhere here);
//   * last commit: NVFP4 needs its scale tensors (a null scale pointer is rejected);
//   * commit on JIT scalars: errors name the offending argument.
// [XQA] "Support NVFP4 KV cache decode on SM120", review: check the capability of
// the device the call runs on, not of a default device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <vector>

#include "internal.h"

using namespace nvfp4;

nvfp4::LaunchEvents& nvfp4::launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

namespace {

thread_local std::string g_error;

nvfp4_status fail(nvfp4_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

nvfp4_status ok() {
  g_error.clear();
  return NVFP4_OK;
}

constexpr size_t kAlign = 256;
constexpr size_t kLdsBytesPerCu = 160 * 1024;  // gfx950
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- device check: gfx950 only, cached per device ordinal.  The device is the one the
// call's stream belongs to (the null stream: the current device), not whatever device
// happens to be current ([XQA] review: the capability check must look at the device the
// tensors are on, not at a default device).
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 gfx950, 2 other

nvfp4_status stream_device(void* stream, int* dev) {
  *dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), dev)
                        : hipGetDevice(dev);
  if (e != hipSuccess || *dev < 0) {
    (void)hipGetLastError();
    return fail(NVFP4_E_DEVICE, stream ? "cannot query the device of the stream: %s"
                                       : "no HIP device is current: %s",
                hipGetErrorString(e));
  }
  return NVFP4_OK;
}

nvfp4_status check_device(void* stream) {
  int dev = -1;
  if (nvfp4_status st = stream_device(stream, &dev)) return st;
  if (dev >= 64) return fail(NVFP4_E_DEVICE, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(NVFP4_E_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (g_dev_state[dev] == 2)
      return fail(NVFP4_E_DEVICE, "device %d is %s, this library needs gfx950", dev,
                  prop.gcnArchName);
  }
  if (g_dev_state[dev] != 1) return fail(NVFP4_E_DEVICE, "device %d is not gfx950", dev);
  return NVFP4_OK;
}

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

// Validates one pool against the expected head dim and shared page geometry.
nvfp4_status check_pool(const nvfp4_kv_pool* p, const char* name, int head_dim,
                        int num_kv_heads, int page_size, int kv_dtype = -1) {
  if (!p) return fail(NVFP4_E_INVALID, "%s pool is NULL", name);
  if (!p->data) return fail(NVFP4_E_INVALID, "%s.data is NULL", name);
  if (p->kv_dtype != NVFP4_KV_NVFP4 && p->kv_dtype != NVFP4_KV_FP8_E4M3)
    return fail(NVFP4_E_INVALID, "%s.kv_dtype %d is neither NVFP4 (0) nor FP8 E4M3 (1)", name,
                p->kv_dtype);
  if (kv_dtype >= 0 && p->kv_dtype != kv_dtype)
    return fail(NVFP4_E_SHAPE, "%s.kv_dtype is %d, the plan was made for %d", name, p->kv_dtype,
                kv_dtype);
  const bool fp8 = p->kv_dtype == NVFP4_KV_FP8_E4M3;
  // [PF] review commit: a scale tensor on a cache that is not NVFP4 is refused rather than
  // silently changing how the cache is read
  if (fp8 && p->sf)
    return fail(NVFP4_E_INVALID, "%s.sf is set on an FP8 pool: FP8 KV has no block scales", name);
  if (!fp8 && !p->sf)
    return fail(NVFP4_E_INVALID, "%s.sf is NULL: NVFP4 needs its scale factors", name);
  if (p->head_dim != head_dim)
    return fail(NVFP4_E_SHAPE, "%s.head_dim is %d, expected %d", name, p->head_dim, head_dim);
  if (num_kv_heads >= 0 && p->num_kv_heads != num_kv_heads)
    return fail(NVFP4_E_SHAPE, "%s.num_kv_heads is %d, expected %d", name, p->num_kv_heads,
                num_kv_heads);
  if (page_size >= 0 && p->page_size != page_size)
    return fail(NVFP4_E_SHAPE, "%s.page_size is %d, expected %d", name, p->page_size, page_size);
  if (!is_pow2(p->page_size) || p->page_size > 256)
    return fail(NVFP4_E_UNSUPPORTED, "%s.page_size %d is not a power of two in [1, 256]", name,
                p->page_size);
  if (p->num_pages < 1) return fail(NVFP4_E_INVALID, "%s.num_pages must be >= 1", name);
  if (p->num_kv_heads < 1) return fail(NVFP4_E_INVALID, "%s.num_kv_heads must be >= 1", name);
  if (!(p->global_scale > 0.f) || !std::isfinite(p->global_scale))
    return fail(NVFP4_E_INVALID, "%s.global_scale must be finite and > 0", name);
  const int64_t da = fp8 ? 16 : (head_dim >= 128 ? 16 : head_dim / 8);
  const int64_t sa = std::min(head_dim / 16, 8);
  if (!aligned(p->data, da) || p->stride_page % da || p->stride_head % da || p->stride_token % da)
    return fail(NVFP4_E_SHAPE, "%s data pointer and strides must be multiples of %lld bytes", name,
                (long long)da);
  if (!fp8 && (!aligned(p->sf, sa) || p->sf_stride_page % sa || p->sf_stride_head % sa ||
               p->sf_stride_token % sa))
    return fail(NVFP4_E_SHAPE, "%s sf pointer and strides must be multiples of %lld bytes", name,
                (long long)sa);
  if (p->stride_page < 0 || p->stride_head < 0 || p->stride_token < 0 ||
      (!fp8 && (p->sf_stride_page < 0 || p->sf_stride_head < 0 || p->sf_stride_token < 0)))
    return fail(NVFP4_E_SHAPE, "%s strides must be non-negative", name);
  const int64_t kMaxStride = (int64_t(1) << 31) - 1;  // kernels multiply strides in 32 bits
  if (p->stride_page > kMaxStride || p->stride_head > kMaxStride || p->stride_token > kMaxStride ||
      (!fp8 && (p->sf_stride_page > kMaxStride || p->sf_stride_head > kMaxStride ||
                p->sf_stride_token > kMaxStride)))
    return fail(NVFP4_E_SHAPE, "%s strides must be below 2^31 bytes", name);
  // the streaming copies address 16 consecutive token slots from one base with a 32-bit
  // offset per lane
  const int64_t kMaxTokStride = int64_t(1) << 27;
  if (p->stride_token >= kMaxTokStride || (!fp8 && p->sf_stride_token >= kMaxTokStride))
    return fail(NVFP4_E_SHAPE, "%s token strides must be below 2^27 bytes", name);
  return NVFP4_OK;
}

PoolArgs pool_args(const nvfp4_kv_pool* p, int num_pages) {
  PoolArgs a;
  a.data = static_cast<const uint8_t*>(p->data);
  a.s_page = p->stride_page;
  a.s_head = p->stride_head;
  a.s_tok = p->stride_token;
  a.sf = static_cast<const uint8_t*>(p->sf);
  a.sf_page = p->sf_stride_page;
  a.sf_head = p->sf_stride_head;
  a.sf_tok = p->sf_stride_token;
  a.num_pages = num_pages;
  return a;
}

}  // namespace

// ---------------------------------------------------------------------------- plan
struct nvfp4_plan {
  int prefill = 0;
  int batch = 0, num_qo_heads = 0, num_kv_heads = 0, group = 0;
  int head_dim_qk = 0, head_dim_vo = 0, page_size = 0, causal = 0;
  int kv_dtype = NVFP4_KV_NVFP4;
  int custom_mask = 0;     // prefill with a packed custom mask (nvfp4_batch_prefill_masked)
  std::vector<int64_t> mask_off;  // byte offset of each request's mask segment
  int64_t mask_bytes = 0;
  int ragged = 0;          // prefill over ragged rows (nvfp4_batch_prefill_ragged)
  std::vector<int32_t> kv_starts;  // ragged: first row of each request
  std::vector<int32_t> ragged_pt;  // ragged: the 16-row "pages" of each request
  int ragged_pt_stride = 0;
  int rope = 0;            // prefill with in-kernel RoPE
  std::vector<float> rope_freq;  // (hi, lo) of w_i / (2 pi) per pair i < Dk/2
  int chunk = 0;           // chunk length used when splitting (0: no split)
  int rows_per_item = 0;   // decode: 16 heads; prefill: rows of a tile
  int rows_per_slot = 0;
  int64_t total_q = 0;
  std::vector<int32_t> work;    // kWorkFields per item
  std::vector<int32_t> merges;  // kMergeFields per merge
  std::vector<int32_t> kv_lens, qo_indptr;
  int num_partials = 0;
  // workspace layout (byte offsets)
  size_t off_work = 0, off_merge = 0, off_kvlens = 0, off_indptr = 0, off_pt = 0, off_mask = 0,
         off_rope = 0, off_part_o = 0, off_part_lse = 0, off_part_scale = 0, ws_bytes = 0;
  std::vector<uint8_t> image;  // the tables as they sit at the start of the workspace
  void* uploaded_to = nullptr;
  int defer_merge = 0;  // runs leave split rows' partials for nvfp4_merge_partials
};

extern "C" {

const char* nvfp4_last_error(void) { return g_error.c_str(); }

const char* nvfp4_version(void) { return "nvfp4_attn 0.1 (gfx950)"; }

nvfp4_status nvfp4_plan_create(const int32_t* kv_lens, const int32_t* qo_indptr, int32_t batch,
                               int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                               int32_t head_dim_vo, int32_t page_size, int32_t causal,
                               int32_t kv_chunk_tokens, int32_t num_cus, nvfp4_plan** out) {
  return nvfp4_plan_create_ex(kv_lens, qo_indptr, batch, num_qo_heads, num_kv_heads, head_dim_qk,
                              head_dim_vo, page_size, causal, kv_chunk_tokens, num_cus, nullptr,
                              out);
}

nvfp4_status nvfp4_plan_create_ex(const int32_t* kv_lens, const int32_t* qo_indptr,
                                  int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                  int32_t head_dim_qk, int32_t head_dim_vo, int32_t page_size,
                                  int32_t causal, int32_t kv_chunk_tokens, int32_t num_cus,
                                  const nvfp4_plan_options* options, nvfp4_plan** out) {
  if (!out) return fail(NVFP4_E_INVALID, "out is NULL");
  *out = nullptr;
  const int kv_dtype = options ? options->kv_dtype : NVFP4_KV_NVFP4;
  const int32_t* kv_indptr = options ? options->kv_indptr : nullptr;
  const bool custom_mask = options && options->custom_mask;
  const int pos_encoding = options ? options->pos_encoding : NVFP4_POS_NONE;
  if (pos_encoding != NVFP4_POS_NONE && pos_encoding != NVFP4_POS_ROPE)
    return fail(NVFP4_E_INVALID, "options.pos_encoding %d is neither none (0) nor RoPE (1)",
                pos_encoding);
  const bool rope = pos_encoding == NVFP4_POS_ROPE;
  if (rope) {
    if (!qo_indptr)
      return fail(NVFP4_E_UNSUPPORTED, "in-kernel RoPE runs in the prefill kernels: qo_indptr "
                  "must be given");
    if (custom_mask)
      return fail(NVFP4_E_UNSUPPORTED, "in-kernel RoPE is not combined with custom masks");
    if (!(options->rope_theta > 0.f) || !std::isfinite(options->rope_theta) ||
        !(options->rope_scale > 0.f) || !std::isfinite(options->rope_scale))
      return fail(NVFP4_E_INVALID, "rope_theta %g and rope_scale %g must be positive and finite",
                  (double)options->rope_theta, (double)options->rope_scale);
  }
  if (custom_mask && !qo_indptr)
    return fail(NVFP4_E_SHAPE, "a custom mask is a prefill mask: qo_indptr must be given");
  if (custom_mask && kv_indptr)
    return fail(NVFP4_E_UNSUPPORTED, "custom masks run over paged KV only, not ragged rows");
  // the mask decides visibility: every tile covers its request's whole key range
  if (custom_mask) causal = 0;
  if (kv_dtype != NVFP4_KV_NVFP4 && kv_dtype != NVFP4_KV_FP8_E4M3)
    return fail(NVFP4_E_INVALID, "options.kv_dtype %d is neither NVFP4 (0) nor FP8 E4M3 (1)",
                kv_dtype);
  if (kv_indptr && !qo_indptr)
    return fail(NVFP4_E_SHAPE, "ragged KV (options.kv_indptr) is a prefill layout: qo_indptr "
                "must be given");
  // ragged rows are streamed as 16-row pages of the row array
  if (kv_indptr) page_size = 16;
  if (batch < 0) return fail(NVFP4_E_INVALID, "batch must be >= 0");
  if (batch > 0 && !kv_lens) return fail(NVFP4_E_INVALID, "kv_lens is NULL");
  if (num_qo_heads < 1 || num_kv_heads < 1)
    return fail(NVFP4_E_INVALID, "num_qo_heads and num_kv_heads must be >= 1");
  if (num_qo_heads % num_kv_heads)
    return fail(NVFP4_E_SHAPE, "num_qo_heads %d is not a multiple of num_kv_heads %d",
                num_qo_heads, num_kv_heads);
  if (!head_dim_ok(head_dim_qk) || !head_dim_ok(head_dim_vo))
    return fail(NVFP4_E_UNSUPPORTED, "head dims (qk %d, vo %d): each must be 64, 128, 256 or 512",
                head_dim_qk, head_dim_vo);
  const bool prefill = qo_indptr != nullptr;
  if (!is_pow2(page_size) || page_size > 256)
    return fail(NVFP4_E_UNSUPPORTED, "page_size %d is not a power of two in [1, 256]", page_size);
  if (head_dim_vo > head_dim_qk)
    return fail(NVFP4_E_UNSUPPORTED, "head dims (qk %d, vo %d) not supported (need vo <= qk)",
                head_dim_qk, head_dim_vo);
  // on-chip budget ([PF] commit "Re-enable split-KV...": a tile that does not fit the
  // on-chip memory is rejected at plan time): the LDS the resident workgroups of this
  // shape's kernel need, then the register file
  const size_t lds = prefill ? prefill_lds_bytes(head_dim_qk, head_dim_vo, page_size, kv_dtype)
                             : decode_lds_bytes(head_dim_qk, head_dim_vo, page_size, kv_dtype);
  if (lds > kLdsBytesPerCu)
    return fail(NVFP4_E_LDS_BUDGET, "%s tile for head dims (%d, %d) needs %zu bytes of LDS per CU, "
                "more than the %zu a CU has", prefill ? "prefill" : "decode", head_dim_qk,
                head_dim_vo, lds, kLdsBytesPerCu);
  if (head_dim_qk == 512 && head_dim_vo == 512)
    return fail(NVFP4_E_LDS_BUDGET,
                "head dims (512, 512): the per-wave decode tile does not fit the register file");
  if (prefill ? !prefill_supported(head_dim_qk, head_dim_vo, kv_dtype)
              : !decode_supported(head_dim_qk, head_dim_vo, kv_dtype))
    return fail(NVFP4_E_UNSUPPORTED, "head dims (qk %d, vo %d) not supported for %s KV",
                head_dim_qk, head_dim_vo, kv_dtype == NVFP4_KV_FP8_E4M3 ? "FP8" : "NVFP4");
  if (kv_chunk_tokens > 0 && kv_chunk_tokens % 16)
    return fail(NVFP4_E_INVALID, "kv_chunk_tokens %d is not a multiple of 16", kv_chunk_tokens);
  if (num_cus < 0) return fail(NVFP4_E_INVALID, "num_cus must be >= 0");
  const int group = num_qo_heads / num_kv_heads;
  if (!prefill && group > 4 * kDecodeHeads)
    return fail(NVFP4_E_UNSUPPORTED, "decode supports at most %d qo heads per kv head, got %d",
                4 * kDecodeHeads, group);
  int rows_item =
      prefill ? prefill_rows_per_item(head_dim_qk, head_dim_vo, group, page_size) : kDecodeHeads;
  if (prefill && group > rows_item)
    return fail(NVFP4_E_UNSUPPORTED, "prefill supports at most %d qo heads per kv head, got %d",
                rows_item, group);

  for (int b = 0; b < batch; ++b) {
    if (kv_lens[b] < 0) return fail(NVFP4_E_INVALID, "kv_lens[%d] = %d is negative", b, kv_lens[b]);
    if (rope && kv_lens[b] > (1 << 24))
      return fail(NVFP4_E_UNSUPPORTED, "kv_lens[%d] = %d: in-kernel RoPE takes positions below "
                  "2^24", b, kv_lens[b]);
  }
  int64_t total_q = batch;
  if (prefill) {
    if (qo_indptr[0] != 0) return fail(NVFP4_E_SHAPE, "qo_indptr[0] must be 0");
    for (int b = 0; b < batch; ++b) {
      const int q = qo_indptr[b + 1] - qo_indptr[b];
      if (q < 0) return fail(NVFP4_E_SHAPE, "qo_indptr is not non-decreasing at %d", b);
      if (q > kv_lens[b])
        return fail(NVFP4_E_SHAPE, "request %d has %d queries but only %d keys", b, q, kv_lens[b]);
    }
    total_q = qo_indptr[batch];
  }
  if (kv_indptr) {
    if (kv_indptr[0] < 0) return fail(NVFP4_E_SHAPE, "kv_indptr[0] must be >= 0");
    for (int b = 0; b < batch; ++b)
      if ((int64_t)kv_indptr[b + 1] - kv_indptr[b] != kv_lens[b])
        return fail(NVFP4_E_SHAPE, "kv_indptr[%d + 1] - kv_indptr[%d] = %lld differs from "
                    "kv_lens[%d] = %d", b, b, (long long)kv_indptr[b + 1] - kv_indptr[b], b,
                    kv_lens[b]);
  }

  if (num_cus == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      num_cus = cus;
    else
      num_cus = 256;
    (void)hipGetLastError();
  }

  auto* plan = new nvfp4_plan();
  plan->prefill = prefill;
  plan->batch = batch;
  plan->num_qo_heads = num_qo_heads;
  plan->num_kv_heads = num_kv_heads;
  plan->group = group;
  plan->head_dim_qk = head_dim_qk;
  plan->head_dim_vo = head_dim_vo;
  plan->page_size = page_size;
  plan->causal = prefill ? (causal != 0) : 0;
  plan->kv_dtype = kv_dtype;
  if (custom_mask) {
    // each request's bits packed on their own, padded to a byte
    plan->custom_mask = 1;
    plan->mask_off.resize(batch);
    int64_t at = 0;
    for (int b = 0; b < batch; ++b) {
      plan->mask_off[b] = at;
      at += ((int64_t)(qo_indptr[b + 1] - qo_indptr[b]) * kv_lens[b] + 7) / 8;
    }
    plan->mask_bytes = at;
    if (at >= (int64_t(1) << 31) - 64) {
      delete plan;
      return fail(NVFP4_E_UNSUPPORTED, "the packed mask would hold %lld bytes; the kernels "
                  "address it with 32-bit offsets", (long long)at);
    }
  }
  if (kv_indptr) {
    // request b's page i starts at row kv_indptr[b] + 16 i: with the page stride equal to
    // the row stride, slot t of that page is row kv_indptr[b] + 16 i + t
    plan->ragged = 1;
    plan->kv_starts.assign(kv_indptr, kv_indptr + batch);
    int maxp = 1;
    for (int b = 0; b < batch; ++b) maxp = std::max(maxp, (kv_lens[b] + 15) / 16);
    plan->ragged_pt_stride = maxp;
    plan->ragged_pt.assign((size_t)batch * maxp, 0);
    for (int b = 0; b < batch; ++b)
      for (int i = 0; i < maxp; ++i)
        plan->ragged_pt[(size_t)b * maxp + i] = kv_indptr[b] + 16 * std::min(i, std::max(0, (kv_lens[b] + 15) / 16 - 1));
  }
  if (rope) {
    // w_i = theta^(-2i/Dk) / scale, in turns per position, split into a float pair
    // whose sum carries it to about 48 bits (the kernels reduce pos * w_i to a fraction
    // of a turn with it)
    plan->rope = 1;
    const int half = head_dim_qk / 2;
    plan->rope_freq.resize(2 * (size_t)half);
    const double two_pi = 6.283185307179586476925286766559;
    for (int i = 0; i < half; ++i) {
      const double w = std::pow((double)options->rope_theta, -2.0 * i / head_dim_qk) /
                       (double)options->rope_scale;
      const double f = w / two_pi;
      const float hi = (float)f;
      plan->rope_freq[2 * i] = hi;
      plan->rope_freq[2 * i + 1] = (float)(f - (double)hi);
    }
  }
  plan->total_q = total_q;
  plan->kv_lens.assign(kv_lens, kv_lens + batch);
  if (prefill) plan->qo_indptr.assign(qo_indptr, qo_indptr + batch + 1);

  // Row groups: decode -> (b, kv head, head block of <= 16 heads) over [0, L);
  // prefill -> (b, kv head, query tile) over the tile's visible key range.
  struct RowGroup {
    int b, kvh, row0, rows, kv_end;
  };
  std::vector<RowGroup> groups;
  if (!prefill) {
    const int nhb = (group + kDecodeHeads - 1) / kDecodeHeads;
    for (int b = 0; b < batch; ++b)
      for (int g = 0; g < num_kv_heads; ++g)
        for (int hb = 0; hb < nhb; ++hb)
          groups.push_back({b, g, hb * kDecodeHeads, std::min(kDecodeHeads, group - hb * kDecodeHeads),
                            kv_lens[b]});
    plan->rows_per_item = kDecodeHeads;
    plan->rows_per_slot = kDecodeHeads;
  } else {
    const int tq = rows_item / group;  // queries per tile
    for (int b = 0; b < batch; ++b) {
      const int qlen = qo_indptr[b + 1] - qo_indptr[b];
      const int L = kv_lens[b];
      for (int g = 0; g < num_kv_heads; ++g)
        for (int q0 = 0; q0 < qlen; q0 += tq) {
          const int qn = std::min(tq, qlen - q0);
          const int end = plan->causal ? std::min(L, q0 + qn - 1 + (L - qlen) + 1) : L;
          groups.push_back({b, g, q0, qn, end});
        }
    }
    plan->rows_per_item = tq * group;
    plan->rows_per_slot = tq * group;
  }

  // Chunk length.  Decode: keys per wave of a whole work item; a work item (one
  // workgroup of four waves) covers four consecutive chunks of a row group, or the
  // whole row when nothing is split, spread evenly over its waves.  Prefill: keys per
  // work item.  Explicit, never, or chosen so that the device is filled: decode aims at
  // as many waves per CU as its kernel keeps resident for this shape, prefill at one
  // and a half rounds of the workgroups its kernel keeps resident.
  int chunk = 0;
  int64_t total = 0;
  int max_len = 0;
  for (const auto& g : groups) {
    total += g.kv_end;
    max_len = std::max(max_len, g.kv_end);
  }
  const int per_item = prefill ? 1 : 4;  // chunks per work item
  if (kv_chunk_tokens > 0) {
    chunk = kv_chunk_tokens;
  } else if (kv_chunk_tokens == 0) {
    // items (prefill) / waves (decode)
    // prefill: one and a half rounds of the resident workgroups, so that the tail
    // round is made of the short chunks
    const int64_t target =
        prefill ? (int64_t)num_cus * prefill_wgs_per_cu(head_dim_qk, head_dim_vo) * 3 / 2
                : (int64_t)num_cus * 4 * decode_wgs_per_cu(head_dim_qk, head_dim_vo, kv_dtype);
    const int64_t have = (int64_t)groups.size() * (prefill ? 1 : 4);
    if (have < target) {
      int64_t c = (total + target - 1) / std::max<int64_t>(target, 1);
      // a prefill chunk amortises its tile's set-up (Q, pipeline fill, partial store
      // and merge) over at least 20 steps
      c = std::max<int64_t>(c, prefill ? 640 : 64);
      c = (c + 31) / 32 * 32;
      if (c * per_item < max_len) chunk = (int)c;
    }
  }
  plan->chunk = chunk;
  const int64_t item_span = chunk > 0 ? (int64_t)chunk * per_item : 0;

  struct Item {
    int32_t f[kWorkFields];
    int len;
  };
  std::vector<Item> items;
  std::vector<int32_t> merges;
  int next_slot = 0;
  for (const auto& g : groups) {
    const int L = g.kv_end;
    const int nitems = (item_span > 0 && L > item_span) ? (int)((L + item_span - 1) / item_span) : 1;
    if (nitems == 1) {
      items.push_back({{g.b, g.kvh, g.row0, g.rows, 0, L, -1, -1}, L});
      continue;
    }
    const int mi = (int)(merges.size() / kMergeFields);
    const int32_t rec[kMergeFields] = {g.b, g.kvh, g.row0, g.rows, next_slot, nitems, 0, 0};
    merges.insert(merges.end(), rec, rec + kMergeFields);
    for (int c = 0; c < nitems; ++c) {
      const int a = (int)(c * item_span), e = (int)std::min<int64_t>(L, (c + 1) * item_span);
      items.push_back({{g.b, g.kvh, g.row0, g.rows, a, e, next_slot + c, mi}, e - a});
    }
    next_slot += nitems;
  }
  // Longest first, so the tail of the grid holds the short items; equal lengths by
  // request, key range, then kv head, so that consecutive workgroups read the heads of
  // the same pages together (a page holds every head's rows in one block).
  std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) {
    if (x.len != y.len) return x.len > y.len;
    if (x.f[W_REQ] != y.f[W_REQ]) return x.f[W_REQ] < y.f[W_REQ];
    if (x.f[W_KV0] != y.f[W_KV0]) return x.f[W_KV0] < y.f[W_KV0];
    return x.f[W_KVH] < y.f[W_KVH];
  });
  plan->work.reserve(items.size() * kWorkFields);
  for (const auto& it : items) plan->work.insert(plan->work.end(), it.f, it.f + kWorkFields);
  plan->merges = std::move(merges);
  plan->num_partials = next_slot;

  // Workspace: [work | merges | kv_lens | qo_indptr | partial O | partial LSE]; everything
  // before the partials is uploaded.
  size_t off = 0;
  plan->off_work = off;
  off = align_up(off + plan->work.size() * sizeof(int32_t));
  plan->off_merge = off;
  off = align_up(off + plan->merges.size() * sizeof(int32_t));
  plan->off_kvlens = off;
  off = align_up(off + (size_t)batch * sizeof(int32_t));
  plan->off_indptr = off;
  off = align_up(off + (size_t)(batch + 1) * sizeof(int32_t));
  plan->off_pt = off;  // ragged plans: the page table of their rows
  off = align_up(off + plan->ragged_pt.size() * sizeof(int32_t));
  plan->off_mask = off;  // custom-mask plans: the requests' segment offsets
  off = align_up(off + plan->mask_off.size() * sizeof(int64_t));
  plan->off_rope = off;  // RoPE plans: the frequency pairs
  off = align_up(off + plan->rope_freq.size() * sizeof(float));
  plan->off_part_o = off;
  off = align_up(off + (size_t)plan->num_partials * plan->rows_per_slot * head_dim_vo * sizeof(_Float16));
  plan->off_part_lse = off;
  off = align_up(off + (size_t)plan->num_partials * plan->rows_per_slot * sizeof(float));
  plan->off_part_scale = off;
  off = align_up(off + sizeof(float));
  plan->ws_bytes = std::max<size_t>(off, kAlign);
  // the uploaded part of the workspace, built once
  plan->image.assign(plan->off_part_o, 0);
  auto put = [&](size_t at, const std::vector<int32_t>& v) {
    if (!v.empty()) std::memcpy(plan->image.data() + at, v.data(), v.size() * sizeof(int32_t));
  };
  put(plan->off_work, plan->work);
  put(plan->off_merge, plan->merges);
  put(plan->off_kvlens, plan->kv_lens);
  put(plan->off_indptr, plan->qo_indptr);
  put(plan->off_pt, plan->ragged_pt);
  if (!plan->mask_off.empty())
    std::memcpy(plan->image.data() + plan->off_mask, plan->mask_off.data(),
                plan->mask_off.size() * sizeof(int64_t));
  if (!plan->rope_freq.empty())
    std::memcpy(plan->image.data() + plan->off_rope, plan->rope_freq.data(),
                plan->rope_freq.size() * sizeof(float));
  *out = plan;
  return ok();
}

void nvfp4_plan_destroy(nvfp4_plan* plan) { delete plan; }

size_t nvfp4_plan_workspace_bytes(const nvfp4_plan* plan) { return plan ? plan->ws_bytes : 0; }

nvfp4_status nvfp4_plan_get_info(const nvfp4_plan* plan, nvfp4_plan_info* info) {
  if (!plan || !info) return fail(NVFP4_E_INVALID, "plan or info is NULL");
  info->num_work_items = (int32_t)(plan->work.size() / kWorkFields);
  info->num_partials = plan->num_partials;
  info->num_merges = (int32_t)(plan->merges.size() / kMergeFields);
  info->kv_chunk_tokens = plan->chunk;
  info->rows_per_item = plan->rows_per_item;
  info->is_prefill = plan->prefill;
  info->workspace_bytes = (int64_t)plan->ws_bytes;
  return ok();
}

nvfp4_status nvfp4_plan_get_work(const nvfp4_plan* plan, int32_t* out, int64_t capacity) {
  if (!plan || !out) return fail(NVFP4_E_INVALID, "plan or out is NULL");
  const int64_t n = (int64_t)(plan->work.size() / kWorkFields);
  if (capacity < n) return fail(NVFP4_E_INVALID, "capacity %lld < %lld work items",
                                (long long)capacity, (long long)n);
  std::memcpy(out, plan->work.data(), plan->work.size() * sizeof(int32_t));
  return ok();
}

nvfp4_status nvfp4_plan_upload(nvfp4_plan* plan, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!plan) return fail(NVFP4_E_INVALID, "plan is NULL");
  if (!workspace) return fail(NVFP4_E_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(NVFP4_E_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < plan->ws_bytes)
    return fail(NVFP4_E_WORKSPACE, "workspace has %zu bytes, plan needs %zu", workspace_bytes,
                plan->ws_bytes);
  if (nvfp4_status st = check_device(stream)) return st;
  // the plan's table image, in one copy
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!plan->image.empty()) {
    hipError_t e = hipMemcpyAsync(workspace, plan->image.data(), plan->image.size(),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(NVFP4_E_HIP, "plan upload failed: %s", hipGetErrorString(e));
  }
  plan->uploaded_to = workspace;
  return ok();
}

}  // extern "C"

namespace {

nvfp4_status check_run(const nvfp4_plan* plan, bool prefill, const void* q, int64_t q_s_row,
                       int64_t q_s_head, const int32_t* page_table, int64_t pt_stride,
                       const nvfp4_kv_pool* k, const nvfp4_kv_pool* v, float sm_scale,
                       void* ws, size_t ws_bytes, float* o, int64_t o_s_row, int64_t o_s_head,
                       float* lse, void* stream, bool need_upload = true) {
  if (!plan) return fail(NVFP4_E_INVALID, "plan is NULL");
  if (plan->prefill != (int)prefill)
    return fail(NVFP4_E_SHAPE, "plan was made for %s, called for %s",
                plan->prefill ? "prefill" : "decode", prefill ? "prefill" : "decode");
  if (nvfp4_status st = check_pool(k, "k_pool", plan->head_dim_qk, plan->num_kv_heads,
                                   plan->page_size, plan->kv_dtype))
    return st;
  if (nvfp4_status st = check_pool(v, "v_pool", plan->head_dim_vo, plan->num_kv_heads,
                                   plan->page_size, plan->kv_dtype))
    return st;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(NVFP4_E_INVALID, "sm_scale must be finite and > 0");
  const bool any_rows = plan->total_q > 0;
  if (any_rows) {
    if (!q) return fail(NVFP4_E_INVALID, "q is NULL");
    if (!o) return fail(NVFP4_E_INVALID, "o is NULL");
    if (!lse) return fail(NVFP4_E_INVALID, "lse is NULL");
    if (!page_table) return fail(NVFP4_E_INVALID, "page_table is NULL");
  }
  if (!aligned(q, 16) || q_s_row % 8 || q_s_head % 8 || q_s_row < 0 || q_s_head < 0)
    return fail(NVFP4_E_SHAPE, "q rows must be 16-byte aligned (strides multiples of 8 elements)");
  if (!aligned(o, 16) || o_s_row % 4 || o_s_head % 4 || o_s_row < 0 || o_s_head < 0)
    return fail(NVFP4_E_SHAPE, "o rows must be 16-byte aligned (strides multiples of 4 elements)");
  if (!aligned(lse, 4)) return fail(NVFP4_E_SHAPE, "lse must be 4-byte aligned");
  int max_pages = 0;
  for (int b = 0; b < plan->batch; ++b)
    max_pages = std::max(max_pages, (plan->kv_lens[b] + plan->page_size - 1) / plan->page_size);
  if (pt_stride < max_pages)
    return fail(NVFP4_E_SHAPE, "pt_stride %lld is smaller than the %d pages of the longest request",
                (long long)pt_stride, max_pages);
  if (!ws) return fail(NVFP4_E_WORKSPACE, "workspace is NULL");
  if (ws_bytes < plan->ws_bytes)
    return fail(NVFP4_E_WORKSPACE, "workspace has %zu bytes, plan needs %zu", ws_bytes,
                plan->ws_bytes);
  if (need_upload && plan->uploaded_to != ws)
    return fail(NVFP4_E_WORKSPACE, "the plan was not uploaded to this workspace (nvfp4_plan_upload)");
  return check_device(stream);
}

// ---- Allocation-free decode: one fixed scratch array per GPU in place of the caller's
// workspace.  In host code `scratch` names a host-side stand-in, never the device
// memory: its device address is taken once per device (hipGetSymbolAddress, with that
// device current) and only that address is used.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

nvfp4_status scratch_address(void* stream, void** out) {
  int dev = -1;
  if (nvfp4_status st = stream_device(stream, &dev)) return st;
  if (dev >= 64) return fail(NVFP4_E_DEVICE, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) cur = -1;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(NVFP4_E_HIP, "cannot make device %d current to find its scratch array", dev);
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && cur >= 0) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(NVFP4_E_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}

AttnArgs make_args(const nvfp4_plan* plan, const void* q, int64_t q_s_row, int64_t q_s_head,
                   const int32_t* page_table, int64_t pt_stride, const nvfp4_kv_pool* k,
                   const nvfp4_kv_pool* v, float sm_scale, void* ws, float* o, int64_t o_s_row,
                   int64_t o_s_head, float* lse) {
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int num_pages = std::min(k->num_pages, v->num_pages);
  a.q = static_cast<const uint16_t*>(q);
  a.q_s_row = q_s_row;
  a.q_s_head = q_s_head;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.k = pool_args(k, num_pages);
  a.v = pool_args(v, num_pages);
  a.score_scale = sm_scale * 1.4426950408889634f * k->global_scale;
  a.out_scale = v->global_scale;
  a.work = reinterpret_cast<const int32_t*>(w + plan->off_work);
  a.n_work = (int32_t)(plan->work.size() / kWorkFields);
  a.kv_lens = reinterpret_cast<const int32_t*>(w + plan->off_kvlens);
  a.qo_indptr = reinterpret_cast<const int32_t*>(w + plan->off_indptr);
  a.o = o;
  a.o_s_row = o_s_row;
  a.o_s_head = o_s_head;
  a.lse = lse;
  a.part_o = reinterpret_cast<_Float16*>(w + plan->off_part_o);
  a.part_lse = reinterpret_cast<float*>(w + plan->off_part_lse);
  a.part_scale = reinterpret_cast<float*>(w + plan->off_part_scale);
  a.num_qo_heads = plan->num_qo_heads;
  a.group = plan->group;
  a.page_shift = log2i(plan->page_size);
  a.rows_per_slot = plan->rows_per_slot;
  a.causal = plan->causal;
  a.merges = reinterpret_cast<const int32_t*>(w + plan->off_merge);
  // heads within 256 bytes of each other share cache lines / DRAM bursts: keep the
  // heads of one key range on one XCD (decode)
  a.xcd_group = !plan->prefill && (std::min(k->stride_head, v->stride_head) <= 256);
  a.stream_kv = !plan->prefill && !a.xcd_group;
  a.rope = plan->rope ? reinterpret_cast<const float*>(w + plan->off_rope) : nullptr;
  return a;
}

nvfp4_status run(const nvfp4_plan* plan, bool prefill, const void* q, int64_t q_s_row,
                 int64_t q_s_head, const int32_t* page_table, int64_t pt_stride,
                 const nvfp4_kv_pool* k, const nvfp4_kv_pool* v, float sm_scale, void* ws,
                 size_t ws_bytes, float* o, int64_t o_s_row, int64_t o_s_head, float* lse,
                 void* stream, const uint8_t* mask = nullptr) {
  if (nvfp4_status st = check_run(plan, prefill, q, q_s_row, q_s_head, page_table, pt_stride, k,
                                  v, sm_scale, ws, ws_bytes, o, o_s_row, o_s_head, lse, stream))
    return st;
  if (plan->work.empty()) return ok();
  AttnArgs a = make_args(plan, q, q_s_row, q_s_head, page_table, pt_stride, k, v, sm_scale, ws, o,
                         o_s_row, o_s_head, lse);
  if (mask) {
    a.mask = mask;
    a.mask_off = reinterpret_cast<const int64_t*>(static_cast<uint8_t*>(ws) + plan->off_mask);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = prefill ? launch_prefill(plan->head_dim_qk, plan->head_dim_vo, plan->kv_dtype,
                                          a.page_shift, a, s)
                         : launch_decode(plan->head_dim_qk, plan->head_dim_vo, plan->kv_dtype,
                                         a.page_shift, a, s);
  if (e != hipSuccess)
    return fail(NVFP4_E_HIP, "%s launch failed: %s", prefill ? "prefill" : "decode",
                hipGetErrorString(e));
  const int n_merges = (int)(plan->merges.size() / kMergeFields);
  if (n_merges > 0 && !plan->defer_merge) {
    e = launch_merge_partials(a, n_merges, plan->head_dim_vo, plan->prefill, s);
    if (e != hipSuccess) return fail(NVFP4_E_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_batch_decode(const nvfp4_plan* plan, const void* q, int64_t q_stride_req,
                                int64_t q_stride_head, const int32_t* page_table, int64_t pt_stride,
                                const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                                float sm_scale, void* workspace, size_t workspace_bytes, float* o,
                                int64_t o_stride_req, int64_t o_stride_head, float* lse,
                                void* stream) {
  return run(plan, false, q, q_stride_req, q_stride_head, page_table, pt_stride, k_pool, v_pool,
             sm_scale, workspace, workspace_bytes, o, o_stride_req, o_stride_head, lse, stream);
}

nvfp4_status nvfp4_batch_decode_noalloc(const nvfp4_plan* plan, const void* q,
                                        int64_t q_stride_req, int64_t q_stride_head,
                                        const int32_t* page_table, int64_t pt_stride,
                                        const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                                        float sm_scale, float* o, int64_t o_stride_req,
                                        int64_t o_stride_head, float* lse, void* stream) {
  if (!plan) return fail(NVFP4_E_INVALID, "plan is NULL");
  if (plan->ws_bytes > kScratchBytes)
    return fail(NVFP4_E_WORKSPACE, "the plan needs %zu bytes of workspace; the allocation-free "
                "entry point has a fixed %zu (use nvfp4_batch_decode with a workspace)",
                plan->ws_bytes, kScratchBytes);
  // every check of nvfp4_batch_decode, with the scratch array as the workspace
  static float probe[4] __attribute__((aligned(16)));
  if (nvfp4_status st = check_run(plan, false, q, q_stride_req, q_stride_head, page_table,
                                  pt_stride, k_pool, v_pool, sm_scale, probe, kScratchBytes, o,
                                  o_stride_req, o_stride_head, lse, stream, false))
    return st;
  void* ws = nullptr;
  if (nvfp4_status st = scratch_address(stream, &ws)) return st;
  if (plan->work.empty()) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the plan's tables into the scratch array, ordered before the kernels on the stream
  hipError_t e = hipMemcpyAsync(ws, plan->image.data(), plan->image.size(),
                                hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return fail(NVFP4_E_HIP, "plan copy failed: %s", hipGetErrorString(e));
  const AttnArgs a = make_args(plan, q, q_stride_req, q_stride_head, page_table, pt_stride, k_pool,
                               v_pool, sm_scale, ws, o, o_stride_req, o_stride_head, lse);
  e = launch_decode(plan->head_dim_qk, plan->head_dim_vo, plan->kv_dtype, a.page_shift, a, s);
  if (e != hipSuccess) return fail(NVFP4_E_HIP, "decode launch failed: %s", hipGetErrorString(e));
  const int n_merges = (int)(plan->merges.size() / kMergeFields);
  if (n_merges > 0) {  // always merged here: the partials live in the shared scratch
    e = launch_merge_partials(a, n_merges, plan->head_dim_vo, 0, s);
    if (e != hipSuccess) return fail(NVFP4_E_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

nvfp4_status nvfp4_batch_decode_append(const nvfp4_plan* plan, const void* q,
                                       int64_t q_stride_req, int64_t q_stride_head,
                                       const void* k_new, int64_t k_new_stride_req,
                                       int64_t k_new_stride_head, const void* v_new,
                                       int64_t v_new_stride_req, int64_t v_new_stride_head,
                                       const int32_t* page_table, int64_t pt_stride,
                                       const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                                       float sm_scale, void* workspace, size_t workspace_bytes,
                                       float* o, int64_t o_stride_req, int64_t o_stride_head,
                                       float* lse, void* stream) {
  // the checks of the new rows come first (they need no device)
  if (plan && plan->kv_dtype != NVFP4_KV_NVFP4)
    return fail(NVFP4_E_UNSUPPORTED, "the in-launch append writes NVFP4; for an FP8 cache use "
                "nvfp4_quantize_kv, then nvfp4_batch_decode");
  if (plan && !plan->prefill && plan->page_size < 16)
    return fail(NVFP4_E_UNSUPPORTED,
                "page_size %d: the in-place append needs pages of at least 16 tokens "
                "(use nvfp4_quantize_kv, then nvfp4_batch_decode)", plan->page_size);
  bool any_keys = false;
  if (plan)
    for (int b = 0; b < plan->batch; ++b) any_keys |= plan->kv_lens[b] > 0;
  if (any_keys && (!k_new || !v_new)) return fail(NVFP4_E_INVALID, "k_new and v_new must be set");
  if (!aligned(k_new, 16) || k_new_stride_req % 8 || k_new_stride_head % 8 ||
      k_new_stride_req < 0 || k_new_stride_head < 0)
    return fail(NVFP4_E_SHAPE, "k_new rows must be 16-byte aligned (strides multiples of 8)");
  if (!aligned(v_new, 16) || v_new_stride_req % 8 || v_new_stride_head % 8 ||
      v_new_stride_req < 0 || v_new_stride_head < 0)
    return fail(NVFP4_E_SHAPE, "v_new rows must be 16-byte aligned (strides multiples of 8)");
  if (nvfp4_status st = check_run(plan, false, q, q_stride_req, q_stride_head, page_table,
                                  pt_stride, k_pool, v_pool, sm_scale, workspace,
                                  workspace_bytes, o, o_stride_req, o_stride_head, lse, stream))
    return st;
  if (plan->work.empty()) return ok();
  AttnArgs a = make_args(plan, q, q_stride_req, q_stride_head, page_table, pt_stride, k_pool,
                         v_pool, sm_scale, workspace, o, o_stride_req, o_stride_head, lse);
  if (any_keys) {
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.kn_s_req = k_new_stride_req;
    a.kn_s_head = k_new_stride_head;
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.vn_s_req = v_new_stride_req;
    a.vn_s_head = v_new_stride_head;
    a.k_gscale = (double)k_pool->global_scale;
    a.v_gscale = (double)v_pool->global_scale;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_decode(plan->head_dim_qk, plan->head_dim_vo, plan->kv_dtype, a.page_shift,
                               a, s);
  if (e != hipSuccess) return fail(NVFP4_E_HIP, "decode launch failed: %s", hipGetErrorString(e));
  const int n_merges = (int)(plan->merges.size() / kMergeFields);
  if (n_merges > 0 && !plan->defer_merge) {
    e = launch_merge_partials(a, n_merges, plan->head_dim_vo, 0, s);
    if (e != hipSuccess) return fail(NVFP4_E_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

nvfp4_status nvfp4_batch_prefill(const nvfp4_plan* plan, const void* q, int64_t q_stride_tok,
                                 int64_t q_stride_head, const int32_t* page_table,
                                 int64_t pt_stride, const nvfp4_kv_pool* k_pool,
                                 const nvfp4_kv_pool* v_pool, float sm_scale, void* workspace,
                                 size_t workspace_bytes, float* o, int64_t o_stride_tok,
                                 int64_t o_stride_head, float* lse, void* stream) {
  if (plan && plan->ragged)
    return fail(NVFP4_E_SHAPE, "the plan was made for ragged KV: use nvfp4_batch_prefill_ragged");
  if (plan && plan->custom_mask)
    return fail(NVFP4_E_SHAPE, "the plan was made for a custom mask: use "
                "nvfp4_batch_prefill_masked");
  return run(plan, true, q, q_stride_tok, q_stride_head, page_table, pt_stride, k_pool, v_pool,
             sm_scale, workspace, workspace_bytes, o, o_stride_tok, o_stride_head, lse, stream);
}

int64_t nvfp4_plan_mask_bytes(const nvfp4_plan* plan) { return plan ? plan->mask_bytes : 0; }

nvfp4_status nvfp4_batch_prefill_masked(const nvfp4_plan* plan, const void* q,
                                        int64_t q_stride_tok, int64_t q_stride_head,
                                        const int32_t* page_table, int64_t pt_stride,
                                        const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                                        const uint8_t* mask, float sm_scale, void* workspace,
                                        size_t workspace_bytes, float* o, int64_t o_stride_tok,
                                        int64_t o_stride_head, float* lse, void* stream) {
  if (!plan) return fail(NVFP4_E_INVALID, "plan is NULL");
  if (!plan->custom_mask)
    return fail(NVFP4_E_SHAPE, "the plan was made without a custom mask: create it with "
                "options.custom_mask");
  // a plan with work has queries, and then keys (q_b <= kv_len_b), so mask bits
  if (!plan->work.empty() && !mask) return fail(NVFP4_E_INVALID, "mask is NULL");
  return run(plan, true, q, q_stride_tok, q_stride_head, page_table, pt_stride, k_pool, v_pool,
             sm_scale, workspace, workspace_bytes, o, o_stride_tok, o_stride_head, lse, stream,
             mask);
}

nvfp4_status nvfp4_batch_prefill_ragged(const nvfp4_plan* plan, const void* q,
                                        int64_t q_stride_tok, int64_t q_stride_head,
                                        const nvfp4_kv_ragged* k, const nvfp4_kv_ragged* v,
                                        float sm_scale, void* workspace, size_t workspace_bytes,
                                        float* o, int64_t o_stride_tok, int64_t o_stride_head,
                                        float* lse, void* stream) {
  if (!plan) return fail(NVFP4_E_INVALID, "plan is NULL");
  if (!plan->ragged)
    return fail(NVFP4_E_SHAPE, "the plan was made for paged KV: create it with "
                "options.kv_indptr for ragged KV");
  if (!k || !v) return fail(NVFP4_E_INVALID, "k and v must be set");
  // the rows a request's last 16-row page reads past its end must exist (they are read
  // and never used): rows up to kv_indptr[b] + 16 * ceil(kv_len_b / 16)
  int64_t need = 0;
  for (int b = 0; b < plan->batch; ++b)
    need = std::max<int64_t>(need, (int64_t)plan->kv_starts[b] +
                                       16 * (int64_t)((plan->kv_lens[b] + 15) / 16));
  nvfp4_kv_pool pools[2];
  const nvfp4_kv_ragged* src[2] = {k, v};
  const char* names[2] = {"k", "v"};
  for (int i = 0; i < 2; ++i) {
    const nvfp4_kv_ragged* r = src[i];
    if (r->num_rows < need)
      return fail(NVFP4_E_SHAPE, "%s has %lld rows; the plan's requests read rows up to %lld "
                  "(every request's rows rounded up to 16)", names[i], (long long)r->num_rows,
                  (long long)need);
    if (r->num_rows > INT32_MAX)
      return fail(NVFP4_E_SHAPE, "%s has more than 2^31 - 1 rows", names[i]);
    // the rows as a pool of one-row pages with 16 slots: page p, slot t is row p + t
    nvfp4_kv_pool& p = pools[i];
    p.data = r->data;
    p.stride_page = r->stride_row;
    p.stride_head = r->stride_head;
    p.stride_token = r->stride_row;
    p.sf = r->sf;
    p.sf_stride_page = r->sf_stride_row;
    p.sf_stride_head = r->sf_stride_head;
    p.sf_stride_token = r->sf_stride_row;
    p.num_pages = (int32_t)r->num_rows;
    p.page_size = 16;
    p.num_kv_heads = r->num_kv_heads;
    p.head_dim = r->head_dim;
    p.global_scale = r->global_scale;
    p.kv_dtype = r->kv_dtype;
  }
  const int32_t* pt = workspace ? reinterpret_cast<const int32_t*>(
                                      static_cast<uint8_t*>(workspace) + plan->off_pt)
                                : nullptr;
  return run(plan, true, q, q_stride_tok, q_stride_head, pt, plan->ragged_pt_stride, &pools[0],
             &pools[1], sm_scale, workspace, workspace_bytes, o, o_stride_tok, o_stride_head, lse,
             stream);
}

nvfp4_status nvfp4_kv_checksum(const nvfp4_plan* plan, const int32_t* page_table,
                               int64_t pt_stride, const nvfp4_kv_pool* k_pool,
                               const nvfp4_kv_pool* v_pool, void* workspace,
                               size_t workspace_bytes, uint32_t* checksum, void* stream) {
  if (plan && plan->prefill)
    return fail(NVFP4_E_SHAPE, "the checksum streams a decode plan, got a prefill plan");
  if (plan && plan->page_size < 16)
    return fail(NVFP4_E_UNSUPPORTED, "page_size %d: the checksum streams through the decode "
                "rings, which need pages of at least 16 tokens", plan->page_size);
  if (plan && !decode_ring_supported(plan->head_dim_qk, plan->head_dim_vo, plan->kv_dtype))
    return fail(NVFP4_E_UNSUPPORTED, "head dims (%d, %d) %s: the checksum streams through the "
                "decode rings, which this shape has none of", plan->head_dim_qk,
                plan->head_dim_vo, plan->kv_dtype == NVFP4_KV_FP8_E4M3 ? "FP8" : "NVFP4");
  if (plan && plan->batch > 0 && !checksum) return fail(NVFP4_E_INVALID, "checksum is NULL");
  if (!aligned(checksum, 4)) return fail(NVFP4_E_SHAPE, "checksum must be 4-byte aligned");
  // the attention checks, with stand-ins for q, o and lse (never read or written)
  static float dummy[4] __attribute__((aligned(16)));
  if (nvfp4_status st = check_run(plan, false, dummy, 0, 0, page_table, pt_stride, k_pool,
                                  v_pool, 1.f, workspace, workspace_bytes, dummy, 0, 0, dummy,
                                  stream))
    return st;
  AttnArgs a = make_args(plan, dummy, 0, 0, page_table, pt_stride, k_pool, v_pool, 1.f,
                         workspace, nullptr, 0, 0, nullptr);
  a.q = nullptr;
  const hipError_t e = launch_kv_checksum(plan->head_dim_qk, plan->head_dim_vo, plan->kv_dtype, a,
                                          checksum,
                                          plan->batch, plan->num_kv_heads,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NVFP4_E_HIP, "checksum launch failed: %s", hipGetErrorString(e));
  return ok();
}

nvfp4_status nvfp4_set_timing_events(void* start_event, void* stop_event) {
  LaunchEvents& ev = launch_events();
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

nvfp4_status nvfp4_plan_set_deferred_merge(nvfp4_plan* plan, int32_t deferred) {
  if (!plan) return fail(NVFP4_E_INVALID, "plan is NULL");
  plan->defer_merge = deferred != 0;
  return ok();
}

nvfp4_status nvfp4_merge_partials(const nvfp4_plan* plan, void* workspace, size_t workspace_bytes,
                                  float* o, int64_t o_stride_row, int64_t o_stride_head, float* lse,
                                  void* stream) {
  if (!plan) return fail(NVFP4_E_INVALID, "plan is NULL");
  const int n_merges = (int)(plan->merges.size() / kMergeFields);
  if (n_merges == 0) return ok();
  if (!workspace) return fail(NVFP4_E_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < plan->ws_bytes)
    return fail(NVFP4_E_WORKSPACE, "workspace has %zu bytes, plan needs %zu", workspace_bytes,
                plan->ws_bytes);
  if (plan->uploaded_to != workspace)
    return fail(NVFP4_E_WORKSPACE, "the plan was not uploaded to this workspace (nvfp4_plan_upload)");
  if (!o) return fail(NVFP4_E_INVALID, "o is NULL");
  if (!lse) return fail(NVFP4_E_INVALID, "lse is NULL");
  if (!aligned(o, 16) || o_stride_row % 4 || o_stride_head % 4 || o_stride_row < 0 ||
      o_stride_head < 0)
    return fail(NVFP4_E_SHAPE, "o rows must be 16-byte aligned (strides multiples of 4 elements)");
  if (!aligned(lse, 4)) return fail(NVFP4_E_SHAPE, "lse must be 4-byte aligned");
  if (nvfp4_status st = check_device(stream)) return st;
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  uint8_t* w = static_cast<uint8_t*>(workspace);
  a.qo_indptr = reinterpret_cast<const int32_t*>(w + plan->off_indptr);
  a.o = o;
  a.o_s_row = o_stride_row;
  a.o_s_head = o_stride_head;
  a.lse = lse;
  a.part_o = reinterpret_cast<_Float16*>(w + plan->off_part_o);
  a.part_lse = reinterpret_cast<float*>(w + plan->off_part_lse);
  a.part_scale = reinterpret_cast<float*>(w + plan->off_part_scale);
  a.num_qo_heads = plan->num_qo_heads;
  a.group = plan->group;
  a.rows_per_slot = plan->rows_per_slot;
  a.merges = reinterpret_cast<const int32_t*>(w + plan->off_merge);
  const hipError_t e = launch_merge_partials(a, n_merges, plan->head_dim_vo, plan->prefill,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NVFP4_E_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

nvfp4_status nvfp4_merge_states(const float* o_parts, const float* lse_parts, int64_t rows,
                                int32_t num_parts, int32_t heads, int32_t head_dim, float* o,
                                float* lse, void* stream) {
  if (rows < 0) return fail(NVFP4_E_INVALID, "rows must be >= 0");
  if (num_parts < 1) return fail(NVFP4_E_INVALID, "num_parts must be >= 1");
  if (heads < 1) return fail(NVFP4_E_INVALID, "heads must be >= 1");
  if (head_dim < 4 || head_dim % 4 || head_dim > 1024)
    return fail(NVFP4_E_UNSUPPORTED, "head_dim %d must be a multiple of 4 in [4, 1024]", head_dim);
  if (rows == 0) return ok();
  if (!o_parts || !lse_parts || !o || !lse)
    return fail(NVFP4_E_INVALID, "o_parts, lse_parts, o and lse must be non-NULL");
  if (!aligned(o_parts, 16) || !aligned(o, 16) || !aligned(lse_parts, 4) || !aligned(lse, 4))
    return fail(NVFP4_E_SHAPE, "o_parts and o must be 16-byte aligned");
  if (nvfp4_status st = check_device(stream)) return st;
  hipError_t e = launch_merge_states(o_parts, lse_parts, rows, num_parts, heads, head_dim, o, lse,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NVFP4_E_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

nvfp4_status nvfp4_quantize_kv(const void* k_src, int64_t k_stride_token, int64_t k_stride_head,
                               const void* v_src, int64_t v_stride_token, int64_t v_stride_head,
                               int64_t n_tokens, const int64_t* slot_mapping,
                               const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                               void* stream) {
  if (n_tokens < 0) return fail(NVFP4_E_INVALID, "n_tokens must be >= 0");
  const bool do_k = k_src || k_pool;
  const bool do_v = v_src || v_pool;
  if (!do_k && !do_v) return fail(NVFP4_E_INVALID, "nothing to quantise: K and V are both NULL");
  if (do_k && (!k_src || !k_pool)) return fail(NVFP4_E_INVALID, "k_src and k_pool must both be set");
  if (do_v && (!v_src || !v_pool)) return fail(NVFP4_E_INVALID, "v_src and v_pool must both be set");
  if (do_k) {
    if (nvfp4_status st = check_pool(k_pool, "k_pool", k_pool->head_dim, -1, -1, -1)) return st;
    if (!head_dim_ok(k_pool->head_dim))
      return fail(NVFP4_E_UNSUPPORTED, "k_pool.head_dim %d unsupported", k_pool->head_dim);
  }
  if (do_v) {
    if (nvfp4_status st = check_pool(v_pool, "v_pool", v_pool->head_dim, -1, -1, -1)) return st;
    if (!head_dim_ok(v_pool->head_dim))
      return fail(NVFP4_E_UNSUPPORTED, "v_pool.head_dim %d unsupported", v_pool->head_dim);
  }
  if (do_k && do_v && k_pool->page_size != v_pool->page_size)
    return fail(NVFP4_E_SHAPE, "k_pool and v_pool page sizes differ");
  if (do_k && (!aligned(k_src, 16) || k_stride_token % 8 || k_stride_head % 8 ||
               k_stride_token < 0 || k_stride_head < 0))
    return fail(NVFP4_E_SHAPE, "k_src rows must be 16-byte aligned (strides multiples of 8)");
  if (do_v && (!aligned(v_src, 16) || v_stride_token % 8 || v_stride_head % 8 ||
               v_stride_token < 0 || v_stride_head < 0))
    return fail(NVFP4_E_SHAPE, "v_src rows must be 16-byte aligned (strides multiples of 8)");
  if (n_tokens == 0) return ok();
  if (!slot_mapping) return fail(NVFP4_E_INVALID, "slot_mapping is NULL");
  if (nvfp4_status st = check_device(stream)) return st;
  auto qa = [](const void* src, int64_t st, int64_t sh, const nvfp4_kv_pool* p) {
    QuantArgs a;
    a.fp8 = p->kv_dtype == NVFP4_KV_FP8_E4M3;
    a.src = static_cast<const uint16_t*>(src);
    a.s_tok = st;
    a.s_head = sh;
    a.data = static_cast<uint8_t*>(p->data);
    a.d_page = p->stride_page;
    a.d_head = p->stride_head;
    a.d_tok = p->stride_token;
    a.sf = static_cast<uint8_t*>(p->sf);
    a.sf_page = p->sf_stride_page;
    a.sf_head = p->sf_stride_head;
    a.sf_tok = p->sf_stride_token;
    a.num_slots = (int64_t)p->num_pages * p->page_size;
    a.page_shift = log2i(p->page_size);
    a.num_heads = p->num_kv_heads;
    a.head_dim = p->head_dim;
    a.gscale = (double)p->global_scale;
    return a;
  };
  QuantArgs ka, va;
  if (do_k) ka = qa(k_src, k_stride_token, k_stride_head, k_pool);
  if (do_v) va = qa(v_src, v_stride_token, v_stride_head, v_pool);
  hipError_t e = launch_quantize(do_k ? &ka : nullptr, do_v ? &va : nullptr, n_tokens,
                                 slot_mapping, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NVFP4_E_HIP, "quantize launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
