/*
 * nvfp4_attn.h -- C ABI for batched attention over a paged KV cache stored as
 * NVFP4, on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [PF]  "Re-enable split-KV for NVFP4 KV cache in prefill path"
 *         (jethac/flashinfer pull request 1, a series of commit messages)
 *   [XQA] "Support NVFP4 KV cache decode on SM120"
 *         (flashinfer-ai/flashinfer pull request 2520)
 *   [FIX] "fix(attention): correct SM120 NVFP4 qk_correction layout, row-sum
 *         reduction, and lse" (flashinfer-ai/flashinfer pull request 3838)
 *
 * Storage format ([PF] commit "Gate split-KV off when kv_data_type is NVFP4";
 * [XQA] changelog): every K or V row of one token and one kv head is packed
 * uint8, two e2m1 values per byte (element 2j in the low nibble of byte j,
 * element 2j+1 in the high nibble), with one FP8 e4m3fn scale byte per 16
 * consecutive head-dim elements.  dequantised value = e2m1 * e4m3 * global_scale.
 * The other 1-byte KV type the same plan serves ([PF] commit "Gate split-KV off...":
 * FP8 and 16-bit KV run the same prefill plan; dtype-aware-skip commit: the
 * float8_e4m3fn KV cache) is FP8: one e4m3fn byte per element, no block scales,
 * dequantised value = e4m3 * global_scale (NVFP4_KV_FP8_E4M3).
 *
 * Conventions shared by every entry point:
 *   - Pointers named "device" are device memory the caller owns (for example
 *     allocated through PyTorch).  The library never allocates device memory and
 *     never frees caller memory.  Pointers named "host" are host memory.
 *   - Every call that takes `stream` (a hipStream_t; NULL = the null stream) is
 *     asynchronous on that stream unless stated otherwise.
 *   - All strides are in the units stated next to them (bytes for the packed
 *     pools, elements for bf16 and fp32 tensors).
 *   - A call that returns anything but NVFP4_OK has launched nothing and written
 *     no output ([PF] commit "Re-enable split-KV...": reject a configuration
 *     cleanly instead of failing later).  nvfp4_last_error() then names the
 *     offending argument.
 *   - Kernels treat a page-table entry outside [0, num_pages) as corrupt input:
 *     they read nothing through it and write NaN to the affected output rows.
 *   - Calls that launch check that the device the stream belongs to (the current
 *     device for the null stream) is a gfx950; the pointers must be memory of that
 *     device ([XQA] review: the check must use the tensors' device, not a default).
 */
#ifndef NVFP4_ATTN_H
#define NVFP4_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_E_INVALID = 1,     /* an argument has an invalid value (null pointer, bad size) */
  NVFP4_E_SHAPE = 2,       /* shapes, strides or alignment inconsistent; plan/run mismatch */
  NVFP4_E_UNSUPPORTED = 3, /* head dim, group size or page size outside the supported set */
  NVFP4_E_LDS_BUDGET = 4,  /* a kernel tile for this shape does not fit on chip: the LDS its
                              resident workgroups need exceeds a CU's 160 KiB, or (head dims
                              512/512) its decode tile exceeds the register file */
  NVFP4_E_WORKSPACE = 5,   /* workspace null, too small, misaligned or not uploaded */
  NVFP4_E_DEVICE = 6,      /* the device of the call's stream is not gfx950 */
  NVFP4_E_HIP = 7          /* a HIP runtime call failed */
} nvfp4_status;

/* Storage type of a K or V pool. */
typedef enum {
  NVFP4_KV_NVFP4 = 0,    /* packed e2m1 pairs + one e4m3 scale byte per 16 elements */
  NVFP4_KV_FP8_E4M3 = 1  /* one e4m3fn byte per element; no scale pool (sf must be NULL) */
} nvfp4_kv_dtype;

/* Text of the last error on the calling thread ("" if none).  Never NULL. */
const char* nvfp4_last_error(void);

/* Library version string. */
const char* nvfp4_version(void);

/*
 * One paged pool: K or V.  K and V have independent pools and independent stride
 * families ([PF] commits on unequal K/V strides: "support-or-reject" contract; this
 * library supports them on every path).  Byte address of packed row
 * (page p, kv head h, token slot t) = data + p*stride_page + h*stride_head +
 * t*stride_token; that row holds head_dim/2 bytes.  Its scale row (head_dim/16
 * bytes) starts at sf + p*sf_stride_page + h*sf_stride_head + t*sf_stride_token.
 * HND and NHD layouts are both expressed through these strides ([XQA] changelog:
 * scale tensors follow the data layout; container strides count bytes).
 * Alignment: data and every data stride must be multiples of 16 bytes when
 * head_dim >= 128 or the pool is FP8, of head_dim/8 bytes otherwise; sf and every sf
 * stride multiples of min(head_dim/16, 8) bytes.  Strides are non-negative and below
 * 2^31 bytes; token strides (data and sf) below 2^27 bytes.  An FP8 pool's rows hold
 * head_dim bytes and it has no scale pool.
 */
typedef struct {
  void* data;              /* device, packed e2m1 pairs (uint8) */
  int64_t stride_page;     /* bytes */
  int64_t stride_head;     /* bytes */
  int64_t stride_token;    /* bytes */
  void* sf;                /* device, e4m3fn scale bytes; required ([PF] last commit: scales
                              are required for NVFP4; [XQA] review: assert scales present) */
  int64_t sf_stride_page;  /* bytes */
  int64_t sf_stride_head;  /* bytes */
  int64_t sf_stride_token; /* bytes */
  int32_t num_pages;       /* pages in the pool; page-table entries must be < num_pages */
  int32_t page_size;       /* tokens per page: a power of two, 1..256 */
  int32_t num_kv_heads;
  int32_t head_dim;        /* 64, 128, 256 or 512 */
  float global_scale;      /* > 0; multiplies every dequantised value */
  int32_t kv_dtype;        /* nvfp4_kv_dtype; NVFP4 pools need sf, FP8 pools must not have it */
} nvfp4_kv_pool;

/*
 * Append (quantise and scatter) K and V rows into their pools ([PF] commit on
 * unequal strides: bf16 sources quantised by the in-tree NVFP4 KV quantisation
 * kernel; [XQA] changelog: to_nvfp4 with a global scale).
 *   k_src, v_src: device bf16 [n_tokens, num_kv_heads, head_dim] with the given
 *     element strides (the last dimension is contiguous and 16-byte aligned).
 *     Either (src, pool) pair may be NULL to quantise only the other.
 *   slot_mapping: device int64 [n_tokens]; token i goes to page slot/page_size,
 *     in-page slot slot%page_size.  A negative slot skips the token; a slot at or
 *     past num_pages*page_size is skipped too.
 * Per 16-element block: s = RNE_e4m3(amax / (6*g)) saturated to 448; element code =
 * RNE_e2m1(|x| / (s*g)), ties to the even code, saturated to 6, sign bit copied
 * from x; s == 0 gives magnitude code 0.  An FP8 pool gets, per element, the sign
 * bit of x and RNE_e4m3(|x| / g) saturated to 448.  Decisions are exact (no rounding
 * of the quotients affects them).  Inputs must be finite.
 */
nvfp4_status nvfp4_quantize_kv(const void* k_src, int64_t k_stride_token, int64_t k_stride_head,
                               const void* v_src, int64_t v_stride_token, int64_t v_stride_head,
                               int64_t n_tokens, const int64_t* slot_mapping,
                               const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                               void* stream);

/*
 * Plan: host-only partition of one batch's attention into work items
 * ([PF] commit "Gate split-KV off...", follow-up: split the KV range with
 * 16-token-aligned chunk boundaries; plan()/run() split of the prefill wrappers;
 * [PF] commits on the smem probe: plan rejects tiles that do not fit).
 *   kv_lens:   host int32 [batch], total keys of each request (>= 0).
 *   qo_indptr: host int32 [batch+1] ragged query offsets for prefill, or NULL for
 *              decode (one query per request).  Prefill requires q_b <= kv_len_b.
 *   causal:    prefill only: query row i of request b sees keys
 *              j <= i + kv_len_b - q_b (bottom-right aligned, prefix extend).
 *   kv_chunk_tokens: 0 = choose the split to fill the device; < 0 = never split;
 *              otherwise a multiple of 16: split every request's KV range into
 *              chunks of that many tokens.  Every chunk boundary except the end of
 *              a request is a multiple of 16 tokens.  A decode work item covers
 *              four consecutive chunks, spread evenly over its four waves in
 *              16-aligned parts (one chunk each when the item is whole) and combined
 *              on chip; a prefill work item covers one chunk; split items are merged
 *              by LSE.
 *   num_cus:   compute units to fill; 0 = query the current device (256 if none).
 * Rejects, with NVFP4_E_LDS_BUDGET, a shape whose kernel's resident workgroups need more
 * LDS than a CU has ([PF] commits on the shared-memory probe: a tile that does not
 * fit on chip is refused at plan time, not at launch).
 * The plan owns host memory only.  It is immutable after creation, except for the
 * record of the workspace it was last uploaded to.
 */
typedef struct nvfp4_plan nvfp4_plan;

nvfp4_status nvfp4_plan_create(const int32_t* kv_lens, const int32_t* qo_indptr, int32_t batch,
                               int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                               int32_t head_dim_vo, int32_t page_size, int32_t causal,
                               int32_t kv_chunk_tokens, int32_t num_cus, nvfp4_plan** out);

/*
 * Options of nvfp4_plan_create_ex ([PF] commit "Gate split-KV off...": one plan()
 * serves the paged and the ragged prefill, over NVFP4 and the other KV types).
 *   kv_dtype:  nvfp4_kv_dtype of the pools the runs read (their kv_dtype must match).
 *              FP8 decode has kernels at every head-dim pair NVFP4 has (512-dim heads
 *              with per-token reads, their rings exceeding the LDS); FP8 prefill up to
 *              256, the 512/256 FP8 prefill tile refused with NVFP4_E_LDS_BUDGET.
 *   kv_indptr: NULL (paged KV), or host int32 [batch+1] for ragged (non-paged) prefill
 *              KV: request b's keys are rows kv_indptr[b] .. kv_indptr[b+1]-1 of one
 *              row array (nvfp4_kv_ragged); kv_indptr[b+1] - kv_indptr[b] must equal
 *              kv_lens[b].  Needs qo_indptr; the page_size argument is then ignored
 *              (the rows stream as 16-row pages), and runs use
 *              nvfp4_batch_prefill_ragged.
 *   custom_mask: prefill (paged KV) whose visibility a packed custom mask decides in
 *              place of the causal rule (nvfp4_batch_prefill_masked); the plan then
 *              tiles every request's whole key range.
 *   pos_encoding: nvfp4_pos_encoding.  NVFP4_POS_ROPE: the prefill kernels rotate Q and
 *              the dequantised K in registers before the QK product ([PF] commit
 *              "Address CodeRabbit review on flashinfer-ai#3684 (5 findings)", item
 *              init_rope_freq: in-kernel RoPE whose frequency table spans half the QK
 *              head dim, also where the VO head dim is smaller).  Rotate-half form:
 *              element i < Dk/2 of a row and element i + Dk/2 turn together by
 *              pos * w_i, w_i = rope_theta^(-2i/Dk) / rope_scale.  Key j of a request
 *              sits at position j (the cache holds un-rotated keys), query row i of a
 *              request with q_b queries and L_b keys at L_b - q_b + i.  Prefill plans
 *              (paged or ragged) only; not with custom_mask (NVFP4_E_UNSUPPORTED for
 *              either), and every kv_len must be at most 2^24 (positions are exact
 *              floats).  V is never rotated.
 *   rope_theta, rope_scale: > 0 and finite when pos_encoding is NVFP4_POS_ROPE
 *              (NVFP4_E_INVALID otherwise); ignored else.
 * A zero-initialised options struct is the plain paged NVFP4 plan.
 */
typedef enum { NVFP4_POS_NONE = 0, NVFP4_POS_ROPE = 1 } nvfp4_pos_encoding;

typedef struct {
  int32_t kv_dtype;
  const int32_t* kv_indptr;
  int32_t custom_mask;  /* nonzero: runs take a packed custom mask (nvfp4_batch_prefill_masked) */
  int32_t pos_encoding; /* nvfp4_pos_encoding */
  float rope_theta;
  float rope_scale;
} nvfp4_plan_options;

/* nvfp4_plan_create with options (NULL options = nvfp4_plan_create). */
nvfp4_status nvfp4_plan_create_ex(const int32_t* kv_lens, const int32_t* qo_indptr,
                                  int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                  int32_t head_dim_qk, int32_t head_dim_vo, int32_t page_size,
                                  int32_t causal, int32_t kv_chunk_tokens, int32_t num_cus,
                                  const nvfp4_plan_options* options, nvfp4_plan** out);

void nvfp4_plan_destroy(nvfp4_plan* plan);

/* Device workspace bytes the runs of this plan need (256-byte aligned). */
size_t nvfp4_plan_workspace_bytes(const nvfp4_plan* plan);

typedef struct {
  int32_t num_work_items;  /* kernel work items (one wave or workgroup each) */
  int32_t num_partials;    /* partial (O, LSE) slots written by split work items */
  int32_t num_merges;      /* row groups merged from partials */
  int32_t kv_chunk_tokens; /* chunk length used (0 when nothing is split) */
  int32_t rows_per_item;   /* query rows x heads covered by one work item (upper bound) */
  int32_t is_prefill;
  int64_t workspace_bytes;
} nvfp4_plan_info;

nvfp4_status nvfp4_plan_get_info(const nvfp4_plan* plan, nvfp4_plan_info* info);

/*
 * Copy the work items as int32 records of 8 fields into host memory `out`
 * (capacity in records): {request, kv_head, row_begin, row_count, kv_begin,
 * kv_end, partial_slot (-1 = written directly), merge_index (-1 = none)}.
 * row_begin/row_count count qo heads within the group (decode) or query rows
 * (prefill).  For tests and tools.
 */
nvfp4_status nvfp4_plan_get_work(const nvfp4_plan* plan, int32_t* out, int64_t capacity);

/*
 * Copy the plan's tables into the workspace (device, >= workspace_bytes, 256-byte
 * aligned) and wait for the copy to finish.  Runs must use a workspace the plan
 * was uploaded to; distinct concurrent runs need distinct workspaces.
 */
nvfp4_status nvfp4_plan_upload(nvfp4_plan* plan, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Decode: one query per request ([XQA] walkthrough: xqa(q, k_cache, v_cache,
 * k_sf_cache, v_sf_cache, page_table, seq_lens, output); [PF] commit on decode
 * strides: K and V addressed through their own strides).
 *   q: device bf16 [batch, num_qo_heads, head_dim_qk], element strides
 *      (last dim contiguous, 16-byte aligned rows).
 *   page_table: device int32 [batch, pt_stride]; entry (b, i) is the page of
 *      tokens [i*page_size, (i+1)*page_size) of request b.
 *   o: device fp32 [batch, num_qo_heads, head_dim_vo] with element strides
 *      (last dim contiguous, 16-byte aligned rows) -- the output is sized by
 *      head_dim_vo ([PF] commits "output sized by VO" / out_head_dim gate).
 *   lse: device fp32 [batch, num_qo_heads] contiguous, natural log, always written
 *      ([PF] commit zeroing lse; [FIX] second commit: ln-sum-exp of the scaled
 *      scores).  A request with kv_len 0 gets O = 0 and LSE = -inf.
 *   sm_scale: finite and > 0; scores are sm_scale * q.k (times the K pool's
 *      global scale).
 * Split work items write partial states into the workspace (each row normalised by its
 * own sum, in fp16, and its LSE; the run also records v_pool's global scale there); a
 * merge kernel on the same stream then combines them by LSE ([XQA] changelog:
 * mergeAndSaveOutTile) and applies the scale, unless the plan defers it
 * (nvfp4_plan_set_deferred_merge).
 */
nvfp4_status nvfp4_batch_decode(const nvfp4_plan* plan, const void* q, int64_t q_stride_req,
                                int64_t q_stride_head, const int32_t* page_table, int64_t pt_stride,
                                const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                                float sm_scale, void* workspace, size_t workspace_bytes, float* o,
                                int64_t o_stride_req, int64_t o_stride_head, float* lse,
                                void* stream);

/*
 * nvfp4_batch_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The library keeps one fixed scratch array of 32 MiB per GPU (a device
 * global, held until the process ends) and uses it as the workspace: each call copies
 * the plan's tables into it on `stream` (the host tables are read before the call
 * returns), then runs the decode and the merge of the split rows.  The call allocates
 * nothing, host or device.
 *   plan: a decode plan whose nvfp4_plan_workspace_bytes is at most 32 MiB
 *     (NVFP4_E_WORKSPACE otherwise); it need not be uploaded.  Its deferred-merge
 *     setting is ignored: split rows are always merged by the call.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents:
 * calls that overlap on one GPU (on different streams, or from different threads
 * without ordering) race and must not be issued.  Other arguments, outputs and errors
 * as for nvfp4_batch_decode.
 */
nvfp4_status nvfp4_batch_decode_noalloc(const nvfp4_plan* plan, const void* q,
                                        int64_t q_stride_req, int64_t q_stride_head,
                                        const int32_t* page_table, int64_t pt_stride,
                                        const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                                        float sm_scale, float* o, int64_t o_stride_req,
                                        int64_t o_stride_head, float* lse, void* stream);

/*
 * Decode with the step's new token appended in the same launch.  For every request b
 * with kv_len_b >= 1, the rows k_new[b] and v_new[b] (device bf16 [batch,
 * num_kv_heads, head_dim_qk / head_dim_vo], element strides, last dim contiguous,
 * 16-byte aligned rows) are quantised exactly as nvfp4_quantize_kv does and written
 * to the slot of token kv_len_b - 1 (its page from the page table), and this call's
 * attention uses them as that key.  The result equals nvfp4_quantize_kv into those
 * slots followed by nvfp4_batch_decode, with one launch less: serving loops append
 * one token per request and attend to it at once ([PF] commit "Gate split-KV off..."
 * and its follow-up describe decode over the growing cache; [XQA] changelog: the
 * tests quantise the cache with to_nvfp4 before decoding).  Requests with kv_len 0
 * append nothing.  Requires page_size >= 16 (NVFP4_E_UNSUPPORTED otherwise).  Other
 * arguments, outputs and errors as for nvfp4_batch_decode.
 */
nvfp4_status nvfp4_batch_decode_append(const nvfp4_plan* plan, const void* q,
                                       int64_t q_stride_req, int64_t q_stride_head,
                                       const void* k_new, int64_t k_new_stride_req,
                                       int64_t k_new_stride_head, const void* v_new,
                                       int64_t v_new_stride_req, int64_t v_new_stride_head,
                                       const int32_t* page_table, int64_t pt_stride,
                                       const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                                       float sm_scale, void* workspace, size_t workspace_bytes,
                                       float* o, int64_t o_stride_req, int64_t o_stride_head,
                                       float* lse, void* stream);

/*
 * Checksum of the paged KV bytes that a decode plan's attention reads, streamed through
 * the same work items, per-wave LDS rings, copies and waits as nvfp4_batch_decode, with
 * no attention arithmetic ([XQA] walkthrough: paged decode streams packed K/V and their
 * scale factors through the page table).  It measures what that access pattern alone
 * sustains, and checks a cache's bytes.
 *   checksum: device uint32 [batch, num_kv_heads]; entry (b, h) = XOR of every 32-bit
 *     little-endian word of the packed K rows, packed V rows, K scale rows and V scale
 *     rows (each row on its own) of tokens [0, kv_len_b) of request b, kv head h; 0 for
 *     kv_len_b = 0.  Written in full (zeroed first) on `stream`.
 * plan: a decode plan (NVFP4_E_SHAPE otherwise) with page_size >= 16 whose head dims
 * have a ring kernel (NVFP4_E_UNSUPPORTED otherwise: FP8 at 512-dim heads decodes with
 * per-token reads instead), uploaded to `workspace`.  Other arguments and errors
 * as for nvfp4_batch_decode.  A page-table entry outside [0, num_pages) reads page 0 in
 * its place (nothing outside the pools is read); that checksum is then meaningless.
 */
nvfp4_status nvfp4_kv_checksum(const nvfp4_plan* plan, const int32_t* page_table,
                               int64_t pt_stride, const nvfp4_kv_pool* k_pool,
                               const nvfp4_kv_pool* v_pool, void* workspace,
                               size_t workspace_bytes, uint32_t* checksum, void* stream);

/*
 * Kernel timing for benchmarks and profilers.  While set, every decode, prefill and
 * checksum launch made by the calling host thread is dispatched with these HIP
 * events (hipEvent_t, cast to void*), which the dispatch itself timestamps when the
 * kernel starts and when it ends (hipExtLaunchKernel), so that their elapsed time is
 * the kernel's own duration without extra queue packets.  The merge and append
 * kernels are not timed.  NULL, NULL stops.  The events belong to the caller and must
 * stay valid while set.  Never fails.
 */
nvfp4_status nvfp4_set_timing_events(void* start_event, void* stop_event);

/*
 * Prefill / extend over the paged cache ([PF] commits on asymmetric heads and
 * "Gate split-KV off...": prefix-cache extend, qo_len << kv_len; causal runs).
 *   q: device bf16 [total_q, num_qo_heads, head_dim_qk] ragged by the plan's
 *      qo_indptr; o: device fp32 [total_q, num_qo_heads, head_dim_vo];
 *   lse: device fp32 [total_q, num_qo_heads] contiguous.
 * A plan made with options.pos_encoding = NVFP4_POS_ROPE applies the rotary embedding
 * to Q and K in the kernels (also nvfp4_batch_prefill_ragged); the rotated rows are
 * never stored.
 * Other arguments as for nvfp4_batch_decode.
 */
nvfp4_status nvfp4_batch_prefill(const nvfp4_plan* plan, const void* q, int64_t q_stride_tok,
                                 int64_t q_stride_head, const int32_t* page_table,
                                 int64_t pt_stride, const nvfp4_kv_pool* k_pool,
                                 const nvfp4_kv_pool* v_pool, float sm_scale, void* workspace,
                                 size_t workspace_bytes, float* o, int64_t o_stride_tok,
                                 int64_t o_stride_head, float* lse, void* stream);

/*
 * Prefill with a packed custom mask ([PF] commits on segment_packbits: packed custom
 * masks for bidirectional, multimodal-prefix attention, built per request segment).
 *   mask: device uint8, the requests' masks packed one after the other: request b's
 *     mask is [q_b, kv_len_b], row-major (query i, key j), bit set = visible; element
 *     e = i*kv_len_b + j is bit e % 8 (little-endian) of byte e / 8 of its segment, and
 *     each segment is padded to a whole byte, so segment b starts at the sum over the
 *     requests before it of ceil(q * kv_len / 8) bytes.  The buffer must be readable 8
 *     bytes past its last segment (nvfp4_plan_mask_bytes() + 8 bytes in all): the
 *     kernels read each query's bits 8 bytes at a time.
 * The mask replaces the causal rule; a query row that sees no key gets O = 0 and
 * LSE = -inf.  plan: made with options.custom_mask (NVFP4_E_SHAPE otherwise; such a
 * plan is refused by nvfp4_batch_prefill).  Other arguments and errors as for
 * nvfp4_batch_prefill.
 */
int64_t nvfp4_plan_mask_bytes(const nvfp4_plan* plan);

nvfp4_status nvfp4_batch_prefill_masked(const nvfp4_plan* plan, const void* q,
                                        int64_t q_stride_tok, int64_t q_stride_head,
                                        const int32_t* page_table, int64_t pt_stride,
                                        const nvfp4_kv_pool* k_pool, const nvfp4_kv_pool* v_pool,
                                        const uint8_t* mask, float sm_scale, void* workspace,
                                        size_t workspace_bytes, float* o, int64_t o_stride_tok,
                                        int64_t o_stride_head, float* lse, void* stream);

/*
 * Ragged (non-paged) K or V rows for nvfp4_batch_prefill_ragged: row r of kv head h
 * starts at data + r*stride_row + h*stride_head (head_dim/2 bytes for NVFP4, head_dim
 * for FP8); NVFP4 scale rows at sf + r*sf_stride_row + h*sf_stride_head.  Strides
 * and alignment as for nvfp4_kv_pool's token and head strides.
 *   num_rows: rows the arrays hold.  Every request's rows are read in 16-row pages,
 *     so the arrays must hold rows up to kv_indptr[b] + 16*ceil(kv_len_b/16) for
 *     every request b (at most 15 rows past the last request, read and never used);
 *     NVFP4_E_SHAPE otherwise.
 */
typedef struct {
  void* data;
  int64_t stride_row;
  int64_t stride_head;
  void* sf;
  int64_t sf_stride_row;
  int64_t sf_stride_head;
  int64_t num_rows;
  int32_t num_kv_heads;
  int32_t head_dim;
  float global_scale;
  int32_t kv_dtype;
} nvfp4_kv_ragged;

/*
 * Prefill / extend over ragged K/V rows ([PF] commit "Gate split-KV off...": the
 * ragged prefill plan beside the paged one).  plan: made with options.kv_indptr
 * (NVFP4_E_SHAPE otherwise; a ragged plan is refused by nvfp4_batch_prefill).  The
 * plan's uploaded workspace holds the rows' page table.  Other arguments, outputs and
 * errors as for nvfp4_batch_prefill.
 */
nvfp4_status nvfp4_batch_prefill_ragged(const nvfp4_plan* plan, const void* q,
                                        int64_t q_stride_tok, int64_t q_stride_head,
                                        const nvfp4_kv_ragged* k, const nvfp4_kv_ragged* v,
                                        float sm_scale, void* workspace, size_t workspace_bytes,
                                        float* o, int64_t o_stride_tok, int64_t o_stride_head,
                                        float* lse, void* stream);

/*
 * Deferred merge ([XQA] changelog: the split-KV partial tiles are merged after the
 * attention pass).  With deferred != 0, nvfp4_batch_decode / nvfp4_batch_prefill
 * runs of this plan write the rows that were not split and leave the split rows'
 * partial states in the workspace; nvfp4_merge_partials then writes those rows'
 * O and LSE (same o, strides and lse as the run), on its stream, after the run.
 * Until it has run, the split rows of o and lse hold nothing meaningful.  Lets a
 * caller place the merge elsewhere on its streams or time the two passes apart.
 * Default: 0 (runs merge by themselves).
 */
nvfp4_status nvfp4_plan_set_deferred_merge(nvfp4_plan* plan, int32_t deferred);

nvfp4_status nvfp4_merge_partials(const nvfp4_plan* plan, void* workspace, size_t workspace_bytes,
                                  float* o, int64_t o_stride_row, int64_t o_stride_head, float* lse,
                                  void* stream);

/*
 * Merge partial attention states by their LSE ([XQA] changelog: merge of the
 * split-KV partial tiles).
 *   o_parts: device fp32 [rows, num_parts, heads, head_dim] contiguous;
 *   lse_parts: device fp32 [rows, num_parts, heads] contiguous (natural log);
 *   o: device fp32 [rows, heads, head_dim]; lse: device fp32 [rows, heads].
 * lse = M + ln sum_c exp(lse_c - M), M = max_c lse_c; o = sum_c exp(lse_c - lse) o_c.
 * Parts with lse = -inf contribute nothing; all -inf gives o = 0, lse = -inf.
 * head_dim: a multiple of 4, at most 1024.
 */
nvfp4_status nvfp4_merge_states(const float* o_parts, const float* lse_parts, int64_t rows,
                                int32_t num_parts, int32_t heads, int32_t head_dim, float* o,
                                float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_ATTN_H */
