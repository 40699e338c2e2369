// Paged NVFP4 decode: one query per request, all qo heads of one kv head together.
//
// [XQA] "Support NVFP4 KV cache decode on SM120", walkthrough: packed K/V and their
// scale factors are streamed through the page table, unpacked, scaled and fed to the
// matrix units; split partials are merged.  [PF] "Re-enable split-KV for NVFP4 KV cache
// in prefill path", commit "Gate split-KV off when kv_data_type is NVFP4" and its
// follow-up: decode splits the KV range into 16-token-aligned chunks whose partial
// states are merged by LSE.  [FIX] "fix(attention): correct SM120 NVFP4 qk_correction
// layout, row-sum reduction, and lse", commits 1-2: a row sum reduces over exactly the
// lanes of that row; lse is ln of the sum of exp of the scaled scores.
//
// A work item is one workgroup of four waves over one key range of one (request,
// kv head, block of <= 16 qo heads).  Wave w takes the w-th 16-aligned quarter of the
// range (one chunk of a full item), streams it in 32-token steps with
// several steps' bytes in flight, and the four states are combined through LDS.  When a
// row group is split over several workgroups, each writes a partial state and a merge
// kernel on the same stream combines them by LSE (a fence-and-counter merge inside this
// kernel was measured slower: each agent-scope release writes back the L2).
#include "fp4_quant.h"
#include "kv_ring.h"

namespace nvfp4 {

namespace {

// Decode reads each K/V byte once per launch: every pool's copies, non-temporal (the
// work records, page table and split partials stay cached; 5-10 % faster measured).
constexpr int kDecodePools = 0xF | kStreamCopies;

// Bytes of one ring workgroup's four rings (0 for shapes without a ring kernel).
template <bool RING, int DK, int DV, int WL, int FMT>
struct RingSmem {
  static constexpr int BYTES = 4 * RingShape<DK, DV, WL, FMT>::WAVE_BYTES;
};
template <int DK, int DV, int WL, int FMT>
struct RingSmem<false, DK, DV, WL, FMT> {
  static constexpr int BYTES = 0;
};

// Workgroups (of four waves) one CU holds at once, by design.  Registers: 512 VGPRs
// per SIMD lane are shared by the waves on a SIMD, and the kernels of each shape are
// held to the budget of this many waves (amdgpu_waves_per_eu).  LDS: 160 KiB per CU,
// and each wave's ring needs two stages at least; a shape whose four waves' rings of
// two stages exceed the LDS (FP8 at 512 dims) has no ring kernel (RING false) and runs
// the register kernel, which needs only the exchange buffer, at every page size.
template <int DK, int DV, int FMT = kNvfp4>
struct DecodeOcc {
  static constexpr int STAGE = RingBytes<DK, DV, FMT>::STAGE;
  static constexpr int BY_REGS = DK <= 128 ? 4 : (DK == 256 && DV <= 128 ? 3 : 2);
  static constexpr int BY_LDS = (160 * 1024) / (4 * 2 * STAGE);
  static constexpr bool RING = BY_LDS > 0;
  // the four waves' states exchanged at the end (accumulators, m, l, bad flag)
  static constexpr int XCH = 3 * (DV / 16 * 4 + 3) * 64 * 4;
  static constexpr int BY_XCH = (160 * 1024) / XCH;
  static constexpr int WGS = RING ? (BY_REGS < BY_LDS ? BY_REGS : BY_LDS)
                                  : (BY_REGS < BY_XCH ? BY_REGS : BY_XCH);
  static constexpr int WAVE_LDS = (160 * 1024) / (4 * WGS);  // one wave's ring budget
  // LDS of one workgroup of the ring kernel: the rings, reused for the exchange
  static constexpr int RING_BYTES = RingSmem<RING, DK, DV, WAVE_LDS, FMT>::BYTES;
  static constexpr int RING_SMEM = RING_BYTES > XCH ? RING_BYTES : XCH;
  static_assert(RING_SMEM * WGS <= 160 * 1024, "resident workgroups exceed the LDS");
  static_assert(XCH * WGS <= 160 * 1024, "resident workgroups exceed the LDS");
};

// Epilogue shared by both decode kernels: combine the four waves' states in wave 0,
// then store the row group directly, or as a partial for the merge kernel.
template <int DV>
__device__ __forceinline__ void decode_epilogue(const AttnArgs& a, RowState<DV / 16, AccForm::VGPR>& st,
                                                float* xch_mem, bool bad_w, int wave, int lane,
                                                int b, int head, int n, int j, bool head_valid,
                                                int slot) {
  constexpr int NT = DV / 16;
  constexpr int NX = NT * 4 + 3;  // per-lane state: accumulators, m, l, bad
  float (*xch)[NX][64] = reinterpret_cast<float (*)[NX][64]>(xch_mem);
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < NT; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) xch[wave - 1][4 * e + i][lane] = st.acc[e][i];
    xch[wave - 1][NX - 3][lane] = st.m;
    xch[wave - 1][NX - 2][lane] = st.l;
    xch[wave - 1][NX - 1][lane] = bad_w ? 1.f : 0.f;
  }
  __syncthreads();
  if (wave > 0) return;
  float bad_any = bad_w ? 1.f : 0.f;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const float m2 = xch[w][NX - 3][lane];
    const float mx = fmaxf(st.m, m2);
    const float mu = mx == -INFINITY ? 0.f : mx;
    const float f1 = fast_exp2(st.m - mu), f2 = fast_exp2(m2 - mu);
#pragma unroll
    for (int e = 0; e < NT; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[e][i] = st.acc[e][i] * f1 + xch[w][4 * e + i][lane] * f2;
    st.l = st.l * f1 + xch[w][NX - 2][lane] * f2;
    st.m = mx;
    bad_any = fmaxf(bad_any, xch[w][NX - 1][lane]);
  }
  const bool bad = bad_any != 0.f;

  float* o_dst = a.o + (int64_t)b * a.o_s_row + (int64_t)head * a.o_s_head;
  float* lse_dst = a.lse + (int64_t)b * a.num_qo_heads + head;
  if (slot < 0) {
    st.store(o_dst, lse_dst, head_valid, bad, a.out_scale, j);
  } else {
    st.store_partial(a.part_o + ((int64_t)slot * a.rows_per_slot + n) * DV,
                     a.part_lse + (int64_t)slot * a.rows_per_slot + n, head_valid, bad, j);
  }
}

// One 32-token step: dequantise K, S^T = K Q^T, online softmax, dequantise V, O^T += V^T P^T.
// MASK: the step may hold keys after tlast.
template <int DK, int DV, bool MASK, int FMT>
__device__ __forceinline__ void decode_step(const StepRaw<DK, DV, FMT>& r, int t0, int tlast, int j,
                                            const f16x8 (&qf)[DK / 32], float score_c,
                                            RowState<DV / 16, AccForm::VGPR>& st) {
  using S = StepShape<DK, DV, FMT>;
  f16x8 ka[S::NS], kb[S::NS];
  k_operands<DK, DV, FMT>(r, ka, kb);
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < S::NS; ++s) {
    sa = mfma16x16x32(ka[s], qf[s], sa);
    sb = mfma16x16x32(kb[s], qf[s], sb);
  }
  const f16x8 p = st.template softmax<MASK>(sa, sb, score_c, t0, j, tlast);
  f16x8 vt[S::NT];
  v_operands<DK, DV, MASK, FMT>(r, t0, tlast, j, vt);
  st.pv(vt, p);
}

// Work record, this wave's key range [w0, w1) and the Q operand: common to both kernels.
struct DecodeItem {
  int b, kvh, h0, hn, kv0, kv1, slot, merge, w0, w1, head;
  bool head_valid;
};

// The work item of this workgroup.  Workgroups are dealt to the eight XCDs in turn
// (workgroup i to XCD i % 8), and the planner puts the kv heads of one key range next
// to each other.  With xcd_group, each full run of 64 workgroups is permuted so that
// eight consecutive items (the heads of one key range) run on one XCD: when the pools
// interleave heads at a short stride (NHD pages, pages of one token) those heads' rows
// share cache lines, which that XCD's L2 then fetches once instead of eight XCDs each.
__device__ __forceinline__ int decode_item_index(const AttnArgs& a) {
  const int bid = blockIdx.x;
  if (!a.xcd_group || bid >= (a.n_work & ~63)) return bid;
  const int r = bid & 63;
  return (bid & ~63) + ((r & 7) << 3) + (r >> 3);
}

__device__ __forceinline__ DecodeItem decode_item(const AttnArgs& a, int wave, int n) {
  const int32_t* rec = a.work + (int64_t)decode_item_index(a) * kWorkFields;
  DecodeItem it;
  it.b = rec[W_REQ]; it.kvh = rec[W_KVH]; it.h0 = rec[W_ROW0]; it.hn = rec[W_ROWS];
  it.kv0 = rec[W_KV0]; it.kv1 = rec[W_KV1]; it.slot = rec[W_SLOT]; it.merge = rec[W_MERGE];
  // the item's keys spread evenly over its four waves, in 16-aligned parts (a full
  // item gives each wave one chunk; a request's shorter last item keeps all four busy)
  const int sub = (((it.kv1 - it.kv0 + 3) / 4 + 15) / 16) * 16;
  it.w0 = min(it.kv1, it.kv0 + wave * sub);
  it.w1 = min(it.kv1, it.w0 + sub);
  it.head_valid = n < it.hn;
  it.head = it.kvh * a.group + it.h0 + n;
  return it;
}

// The step's new token, appended by the wave whose keys end at the request's last key.
// The concatenated K and V rows are quantised four elements per lane: quarter q goes to
// lane q % 64, slot q / 64, and the four lanes of a 16-element block share its largest
// magnitude through two lane exchanges (the arithmetic is the append kernel's).  The
// codes are written to the pools at once and stay in registers until the wave's last
// step, where they replace the token's bytes in the ring: the ring never depends on
// the pool write being visible to the copies.
template <int DK, int DV>
struct NewToken {
  static constexpr int QK = DK / 4;          // quarters of the K row
  static constexpr int QT = (DK + DV) / 4;   // quarters of both rows
  static constexpr int RQ = (QT + 63) / 64;  // per lane
  uint32_t codes[RQ];                        // 16 bits: four e2m1 codes
  uint32_t sc[RQ];                           // the block's e4m3 scale code

  __device__ __forceinline__ void quantise(const AttnArgs& a, int b, int kvh, int lane) {
    const uint16_t* krow = a.k_new + (int64_t)b * a.kn_s_req + (int64_t)kvh * a.kn_s_head;
    const uint16_t* vrow = a.v_new + (int64_t)b * a.vn_s_req + (int64_t)kvh * a.vn_s_head;
#pragma unroll
    for (int r = 0; r < RQ; ++r) {
      const int q = lane + 64 * r;
      uint2 u = make_uint2(0u, 0u);
      if (q < QT) u = *reinterpret_cast<const uint2*>(q < QK ? krow + 4 * q : vrow + 4 * (q - QK));
      float amax = quant::amax4(u.x, u.y);
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      const double gs = q < QK ? a.k_gscale : a.v_gscale;
      sc[r] = quant::scale_code(amax, gs);
      codes[r] = quant::codes4(u.x, u.y, sc[r], gs);
    }
  }

  // Writes the token (step token tt) into the ring stage at byte address `stage`.
  template <int WL>
  __device__ __forceinline__ void inject(uint32_t stage, int tt, int lane) const {
    using R = RingShape<DK, DV, WL>;
    typedef __attribute__((address_space(3))) uint16_t* lds_u16;
    typedef __attribute__((address_space(3))) uint8_t* lds_u8;
#pragma unroll
    for (int r = 0; r < RQ; ++r) {
      const int q = lane + 64 * r;
      if (q >= QT) continue;
      const bool isk = q < QK;
      const int e = isk ? q : q - QK;  // quarter within its row
      const uint32_t row = isk ? R::OFF_KD + tt * (DK / 2) : R::OFF_VD + tt * (DV / 2);
      const uint32_t sf = isk ? R::OFF_SF + tt * (DK / 16) : R::OFF_SF + R::KS + tt * (DV / 16);
      *(lds_u16)(size_t)(stage + row + 2 * e) = (uint16_t)codes[r];
      if ((e & 3) == 0) *(lds_u8)(size_t)(stage + sf + (e >> 2)) = (uint8_t)sc[r];
    }
  }

  // Writes the token (key `tok` of the request) to the pools; an out-of-range page
  // writes nothing (the request's outputs are NaN then).
  __device__ __forceinline__ void store(const PagedView<DK, DV, true>& v, int tok, int lane) const {
    const int pg = v.pt_row[tok >> v.page_shift];
    if ((unsigned)pg >= (unsigned)v.num_pages) return;
    const int64_t sl = tok & v.page_mask;
    uint8_t* kd = const_cast<uint8_t*>(v.kdat) + pg * v.k_page + sl * v.k_tok;
    uint8_t* ks = const_cast<uint8_t*>(v.ksf) + pg * v.ksf_page + sl * v.ksf_tok;
    uint8_t* vd = const_cast<uint8_t*>(v.vdat) + pg * v.v_page + sl * v.v_tok;
    uint8_t* vs = const_cast<uint8_t*>(v.vsf) + pg * v.vsf_page + sl * v.vsf_tok;
#pragma unroll
    for (int r = 0; r < RQ; ++r) {
      const int q = lane + 64 * r;
      // separate guarded blocks for K and V (an if/else pair gets merged into one store
      // through a stack table of pointers)
      if (q < QK) {
        *reinterpret_cast<uint16_t*>(kd + 2 * q) = (uint16_t)codes[r];
        if ((q & 3) == 0) ks[q >> 2] = (uint8_t)sc[r];
      }
      const int e = q - QK;
      if (e >= 0 && q < QT) {
        *reinterpret_cast<uint16_t*>(vd + 2 * e) = (uint16_t)codes[r];
        if ((e & 3) == 0) vs[e >> 2] = (uint8_t)sc[r];
      }
    }
  }
};

// page_size >= 16: the chunk streams through a per-wave LDS ring several steps deep.
// APPEND: the launch also appends the step's new token (AttnArgs::k_new).
template <int DK, int DV, bool APPEND, int FMT = kNvfp4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DecodeOcc<DK, DV, FMT>::WGS)))
void decode_ring_kernel(AttnArgs a) {
  static_assert(!APPEND || FMT == kNvfp4, "the in-launch append writes NVFP4");
  using S = StepShape<DK, DV, FMT>;
  constexpr int WL = DecodeOcc<DK, DV, FMT>::WAVE_LDS;
  using R = RingShape<DK, DV, WL, FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeOcc<DK, DV, FMT>::RING_SMEM];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4;
  const int n = lane & 15;
  const DecodeItem it = decode_item(a, wave, n);
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.part_scale = a.out_scale;  // for the merge

  PagedView<DK, DV, true, FMT> view;
  view.init(a, it.b, it.kvh, lane);
  RingPlan<DK, DV, WL, FMT> rp;
  rp.init(lane, view.k_tok, view.v_tok, view.ksf_tok, view.vsf_tok);
  uint8_t* ring = smem + wave * R::WAVE_BYTES;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ring);
  const int tlast = it.w1 - 1;
  uint32_t bad = 0;

  RingLanes lanes = ring_lanes<DK, DV, WL, FMT>(ring_lds, j, n);
  const int len = it.w1 - it.w0;
  const int nsteps = (len + kDecodeStep - 1) / kDecodeStep;
  // the wave holding the request's last key appends the step's new token; its last
  // step is then always taken by the peeled (masked) code
  const bool appender = APPEND && len > 0 && it.w1 == a.kv_lens[it.b];
  const int nfull = appender ? nsteps - 1 : len / kDecodeStep;  // steps of the unrolled loop
#pragma unroll
  for (int s = 0; s < R::NST - 1; ++s)
    if (s < nsteps)
      ring_issue<DK, DV, WL, kDecodePools>(rp, ring_lds + s * R::STAGE, view,
                                            it.w0 + s * kDecodeStep, tlast, bad);
  // Q (and the new token's rows) after the first copies, so that their loads overlap
  f16x8 qf[S::NS];
  const float score_c = a.score_scale *
      load_q_operand<DK>(a.q + (int64_t)it.b * a.q_s_row + (int64_t)it.head * a.q_s_head,
                         it.head_valid, j, qf);
  NewToken<DK, DV> nt;
  if constexpr (APPEND) if (appender) {
    nt.quantise(a, it.b, it.kvh, lane);
    // Written to the pools now, overlapping the stream.  The stores join the wave's
    // vmcnt queue ahead of later copies, which only makes the ring's waits stronger;
    // the ring itself takes the token's bytes from registers (below).
    nt.store(view, tlast, lane);
  }

  RowState<S::NT, AccForm::VGPR> st;
  st.init();
  // Long chunks: wave priority from the steps a wave has left (longest remaining
  // first).  The waves resident on a CU otherwise share its memory issue oldest first:
  // with one round of equal chunks (the long-context workload, 64 steps per wave) the
  // first-dispatched workgroups finished in 114 us and the last in 200, the early ones'
  // slots idle meanwhile; ranking by the work left evens that out (221 -> 211 us).  Short
  // chunks (the batch workload, 8 steps per wave, 2.3 rounds of work items) keep equal
  // priorities: there a second-round item would overtake the ones about to finish, and it
  // measured 3 % slower.
  const bool lrpt = nsteps >= 24;
  // Full steps, unrolled by the ring depth so that every stage offset is a constant.
  // Step i issues step i + NST - 1 (when it exists) into the stage step i - 1 used,
  // then waits until at most NST - 1 steps are newer than its own.
  for (int i0 = 0; i0 < nfull; i0 += R::NST) {
#pragma unroll
    for (int s = 0; s < R::NST; ++s) {
      const int i = i0 + s;
      if (i >= nfull) break;
      if (lrpt) {
        const int rem = nsteps - i;
        if (rem >= 24) __builtin_amdgcn_s_setprio(3);
        else if (rem >= 12) __builtin_amdgcn_s_setprio(2);
        else if (rem >= 4) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      const int ahead = i + R::NST - 1;
      const bool more = ahead < nsteps;
      if (more)
        ring_issue<DK, DV, WL, kDecodePools>(rp, ring_lds + ((s + R::NST - 1) % R::NST) * R::STAGE,
                                            view, it.w0 + ahead * kDecodeStep, tlast, bad);
      ring_wait_sel<(R::NST - 1) * R::NDMA>(lanes, more);
      StepRaw<DK, DV, FMT> raw;
      ring_read<DK, DV, FMT>(lanes, s * R::STAGE, raw);
      decode_step<DK, DV, false, FMT>(raw, it.w0 + i * kDecodeStep, tlast, j, qf, score_c, st);
    }
  }
  if (nfull < nsteps) {  // the last step: partial, or the appender's; it was issued already
    ring_wait<0>(lanes);
    const uint32_t stage_off = (uint32_t)(nfull % R::NST) * R::STAGE;
    const int t0 = it.w0 + nfull * kDecodeStep;
    if constexpr (APPEND) if (appender) {
      uint32_t stage = ring_lds + stage_off;
      asm volatile("" : "+v"(stage));  // after the wait: the copies have landed
      nt.template inject<WL>(stage, tlast - t0, lane);
    }
    StepRaw<DK, DV, FMT> raw;
    ring_read<DK, DV, FMT>(lanes, stage_off, raw);
    decode_step<DK, DV, true, FMT>(raw, t0, tlast, j, qf, score_c, st);
  }
  const bool bad_w = __any(bad != 0);
  __syncthreads();  // every wave is done with its ring: the exchange reuses that memory
  decode_epilogue<DV>(a, st, reinterpret_cast<float*>(smem), bad_w, wave, lane, it.b, it.head, n,
                      j, it.head_valid, it.slot);
}

// XOR of the 32-bit words this lane's copies placed in a ring stage: K rows, V rows
// (16 bytes per lane and copy) and the scale region (4 bytes per lane and copy, K's
// scales first).  MASK: words of tokens after `tl` (step-relative) are left out.
// dat / sf: this lane's byte address in the data and scale regions of stage 0.
template <int DK, int DV, int WL, bool MASK, int FMT>
__device__ __forceinline__ uint32_t fold_stage(uint32_t dat, uint32_t sf, uint32_t stage_off,
                                               int lane, int tl) {
  using R = RingShape<DK, DV, WL, FMT>;
  uint32_t x = 0;
#pragma unroll
  for (int c = 0; c < R::N_KD; ++c) {
    if (MASK && (c * 1024 + 16 * lane) / R::RBK > tl) continue;
    uint32_t w[4];
    lds_load<16>(dat + stage_off + R::OFF_KD + c * 1024, w);
    x ^= w[0] ^ w[1] ^ w[2] ^ w[3];
  }
#pragma unroll
  for (int c = 0; c < R::N_VD; ++c) {
    if (MASK && (c * 1024 + 16 * lane) / R::RBV > tl) continue;
    uint32_t w[4];
    lds_load<16>(dat + stage_off + R::OFF_VD + c * 1024, w);
    x ^= w[0] ^ w[1] ^ w[2] ^ w[3];
  }
#pragma unroll
  for (int c = 0; c < R::N_SF; ++c) {
    const int byte = c * 256 + 4 * lane;
    if (byte >= R::KS + R::VS) continue;  // padding lanes copy nothing
    const int tok = byte < R::KS ? byte / R::SBK : (byte - R::KS) / R::SBV;
    if (MASK && tok > tl) continue;
    uint32_t w;
    lds_load<4>(sf + stage_off + c * 256, &w);
    x ^= w;
  }
  return x;
}

// Checksum of the KV bytes a decode plan's attention reads, streamed exactly as
// decode_ring_kernel streams them (same work items, rings, copies and waits) and folded
// by XOR instead of attended: the access pattern's own ceiling, with a result that can
// be checked.  out[b * Hkv + h] ^= the XOR of every 32-bit word of the packed K and V
// rows and of their scale rows of the item's keys.  Only the first block of qo heads
// of a row group streams (larger groups repeat the same keys for each block).
template <int DK, int DV, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DecodeOcc<DK, DV, FMT>::WGS)))
void kv_checksum_kernel(AttnArgs a, uint32_t* out, int num_kv_heads) {
  constexpr int WL = DecodeOcc<DK, DV, FMT>::WAVE_LDS;
  using R = RingShape<DK, DV, WL, FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeOcc<DK, DV, FMT>::RING_SMEM];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const DecodeItem it = decode_item(a, wave, lane & 15);
  if (it.h0 != 0) return;  // uniform over the workgroup; no barrier follows
  PagedView<DK, DV, true, FMT> view;
  view.init(a, it.b, it.kvh, lane);
  RingPlan<DK, DV, WL, FMT> rp;
  rp.init(lane, view.k_tok, view.v_tok, view.ksf_tok, view.vsf_tok);
  const uint32_t ring_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(smem + wave * R::WAVE_BYTES));
  const int tlast = it.w1 - 1;
  uint32_t bad = 0;
  // the fold's lane addresses pass through every wait, which orders the reads after it
  RingLanes lanes;
  lanes.k = ring_lds + 16 * lane;
  lanes.ks = ring_lds + R::OFF_SF + 4 * lane;
  lanes.v = lanes.vs = 0;
  const int len = it.w1 - it.w0;
  const int nsteps = (len + kDecodeStep - 1) / kDecodeStep;
  const int nfull = len / kDecodeStep;
#pragma unroll
  for (int s = 0; s < R::NST - 1; ++s)
    if (s < nsteps)
      ring_issue<DK, DV, WL, kDecodePools>(rp, ring_lds + s * R::STAGE, view,
                                            it.w0 + s * kDecodeStep, tlast, bad);
  uint32_t x = 0;
  for (int i0 = 0; i0 < nfull; i0 += R::NST) {
#pragma unroll
    for (int s = 0; s < R::NST; ++s) {
      const int i = i0 + s;
      if (i >= nfull) break;
      const int ahead = i + R::NST - 1;
      const bool more = ahead < nsteps;
      if (more)
        ring_issue<DK, DV, WL, kDecodePools>(rp, ring_lds + ((s + R::NST - 1) % R::NST) * R::STAGE,
                                              view, it.w0 + ahead * kDecodeStep, tlast, bad);
      ring_wait_sel<(R::NST - 1) * R::NDMA>(lanes, more);
      x ^= fold_stage<DK, DV, WL, false, FMT>(lanes.k, lanes.ks, s * R::STAGE, lane, 0);
    }
  }
  if (nfull < nsteps) {
    ring_wait<0>(lanes);
    x ^= fold_stage<DK, DV, WL, true, FMT>(lanes.k, lanes.ks,
                                           (uint32_t)(nfull % R::NST) * R::STAGE, lane,
                                           tlast - (it.w0 + nfull * kDecodeStep));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if (lane == 0 && len > 0) atomicXor(out + (int64_t)it.b * num_kv_heads + it.kvh, x);
}

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// page_size < 16: every token is looked up on its own; the next step is held in registers.
template <int DK, int DV, int FMT = kNvfp4>
__global__ __launch_bounds__(256) void decode_regs_kernel(AttnArgs a) {
  using S = StepShape<DK, DV, FMT>;
  __shared__ float xch[DecodeOcc<DK, DV, FMT>::XCH / 4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4;
  const int n = lane & 15;
  const DecodeItem it = decode_item(a, wave, n);
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.part_scale = a.out_scale;  // for the merge

  f16x8 qf[S::NS];
  const float score_c = a.score_scale *
      load_q_operand<DK>(a.q + (int64_t)it.b * a.q_s_row + (int64_t)it.head * a.q_s_head,
                         it.head_valid, j, qf);
  PagedView<DK, DV, false, FMT> view;
  view.init(a, it.b, it.kvh, lane);
  const int tlast = it.w1 - 1;
  RowState<S::NT, AccForm::VGPR> st;
  st.init();
  const int len = it.w1 - it.w0;
  const int nsteps = (len + kDecodeStep - 1) / kDecodeStep;
  const int nfull = len / kDecodeStep;
  auto t_of = [&](int i) { return it.w0 + i * kDecodeStep; };
  using View = PagedView<DK, DV, false, FMT>;
  // r0 holds step i at the top of every iteration, p1 the pages of step i + 1; full
  // steps in pairs, unmasked.  A step's page-table entries are read one step before its
  // bytes, its bytes one step before its compute.
  StepRaw<DK, DV, FMT> r0, r1;
  typename View::Pages p0, p1;
  if (nsteps > 0) view.load(r0, t_of(0), tlast);
  if (nsteps > 1) view.lookup(p1, t_of(1), tlast);
  int i = 0;
  for (; i + 1 < nfull; i += 2) {
    if (i + 2 < nsteps) view.lookup(p0, t_of(i + 2), tlast);
    view.load(r1, p1, t_of(i + 1), tlast);
    decode_step<DK, DV, false, FMT>(r0, t_of(i), tlast, j, qf, score_c, st);
    if (i + 3 < nsteps) view.lookup(p1, t_of(i + 3), tlast);
    if (i + 2 < nsteps) view.load(r0, p0, t_of(i + 2), tlast);
    decode_step<DK, DV, false, FMT>(r1, t_of(i + 1), tlast, j, qf, score_c, st);
  }
  // at most two steps are left, the second one partial (its pages are in p1)
  if (i < nsteps) {
    if (i + 1 < nsteps) view.load(r1, p1, t_of(i + 1), tlast);
    decode_step<DK, DV, true, FMT>(r0, t_of(i), tlast, j, qf, score_c, st);
    if (i + 1 < nsteps) decode_step<DK, DV, true, FMT>(r1, t_of(i + 1), tlast, j, qf, score_c, st);
  }
  const bool bad_w = __any(view.bad != 0);
  decode_epilogue<DV>(a, st, xch, bad_w, wave, lane, it.b, it.head, n, j, it.head_valid, it.slot);
}

template <int DK, int DV, int FMT>
hipError_t launch_dk_dv(int page_shift, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_work);
  if constexpr (FMT == kNvfp4) {
    if (page_shift >= 4 && a.k_new) {
      launch_attention(decode_ring_kernel<DK, DV, true>, grid, dim3(256), stream, a);
      return hipGetLastError();
    }
  }
  if (a.k_new) return hipErrorInvalidValue;  // the append: NVFP4 with page_size >= 16 only
  if constexpr (DecodeOcc<DK, DV, FMT>::RING) {
    if (page_shift >= 4) {
      launch_attention(decode_ring_kernel<DK, DV, false, FMT>, grid, dim3(256), stream, a);
      return hipGetLastError();
    }
  }
  launch_attention(decode_regs_kernel<DK, DV, FMT>, grid, dim3(256), stream, a);
  return hipGetLastError();
}

}  // namespace

// Shapes with kernels: NVFP4 at every (qk, vo) pair of 64..512 with vo <= qk except
// 512/512; FP8 at the same pairs.  A 512-dim FP8 ring does not fit two stages of four
// waves in LDS, so those shapes run the register kernel at every page size.
#define NVFP4_DECODE_SHAPES(X)                                                      \
  X(64, 64, kNvfp4) X(128, 64, kNvfp4) X(128, 128, kNvfp4) X(256, 64, kNvfp4)      \
  X(256, 128, kNvfp4) X(256, 256, kNvfp4) X(512, 64, kNvfp4) X(512, 128, kNvfp4)   \
  X(512, 256, kNvfp4) X(64, 64, kFp8) X(128, 64, kFp8) X(128, 128, kFp8)           \
  X(256, 64, kFp8) X(256, 128, kFp8) X(256, 256, kFp8) X(512, 64, kFp8)            \
  X(512, 128, kFp8) X(512, 256, kFp8)

bool decode_supported(int dk, int dv, int fmt) {
#define NVFP4_DECODE_CASE(K, V, F) \
  if (dk == K && dv == V && fmt == F) return true;
  NVFP4_DECODE_SHAPES(NVFP4_DECODE_CASE)
#undef NVFP4_DECODE_CASE
  return false;
}

bool decode_ring_supported(int dk, int dv, int fmt) {
#define NVFP4_DECODE_CASE(K, V, F) \
  if (dk == K && dv == V && fmt == F) return DecodeOcc<K, V, F>::RING;
  NVFP4_DECODE_SHAPES(NVFP4_DECODE_CASE)
#undef NVFP4_DECODE_CASE
  return false;
}

int decode_wgs_per_cu(int dk, int dv, int fmt) {
#define NVFP4_DECODE_CASE(K, V, F) \
  if (dk == K && dv == V && fmt == F) return DecodeOcc<K, V, F>::WGS;
  NVFP4_DECODE_SHAPES(NVFP4_DECODE_CASE)
#undef NVFP4_DECODE_CASE
  return 2;
}

size_t decode_lds_bytes(int dk, int dv, int page_size, int fmt) {
  // per CU: the resident workgroups' rings (page_size >= 16) or exchange buffers
#define NVFP4_DECODE_CASE(K, V, F)                                                   \
  if (dk == K && dv == V && fmt == F)                                                \
    return (size_t)DecodeOcc<K, V, F>::WGS *                                         \
           (page_size >= 16 ? DecodeOcc<K, V, F>::RING_SMEM : DecodeOcc<K, V, F>::XCH);
  NVFP4_DECODE_SHAPES(NVFP4_DECODE_CASE)
#undef NVFP4_DECODE_CASE
  // shapes without a kernel: the least a ring workgroup needs (four waves, two stages)
  const int rbk = fmt == kFp8 ? dk : dk / 2, rbv = fmt == kFp8 ? dv : dv / 2;
  const int sf = fmt == kFp8 ? 0 : (2 * dk + 2 * dv + 255) / 256 * 256;
  const size_t stage = (size_t)32 * (rbk + rbv) + sf;
  return page_size >= 16 ? 8 * stage : (size_t)3 * (dv / 16 * 4 + 3) * 64 * 4;
}

hipError_t launch_kv_checksum(int dk, int dv, int fmt, const AttnArgs& a, uint32_t* out,
                              int batch, int num_kv_heads, hipStream_t stream) {
  const int64_t n = (int64_t)batch * num_kv_heads;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     out, n);
  if (a.n_work <= 0) return hipGetLastError();
  const dim3 grid(a.n_work);
#define NVFP4_DECODE_CASE(K, V, F)                                                       \
  if (dk == K && dv == V && fmt == F) {                                                  \
    if constexpr (DecodeOcc<K, V, F>::RING) {                                            \
      launch_attention(kv_checksum_kernel<K, V, F>, grid, dim3(256), stream, a, out,     \
                       num_kv_heads);                                                    \
      return hipGetLastError();                                                          \
    }                                                                                    \
    return hipErrorInvalidValue;                                                         \
  }
  NVFP4_DECODE_SHAPES(NVFP4_DECODE_CASE)
#undef NVFP4_DECODE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int dk, int dv, int fmt, int page_shift, const AttnArgs& a,
                         hipStream_t stream) {
  if (a.n_work <= 0) return hipSuccess;
#define NVFP4_DECODE_CASE(K, V, F) \
  if (dk == K && dv == V && fmt == F) return launch_dk_dv<K, V, F>(page_shift, a, stream);
  NVFP4_DECODE_SHAPES(NVFP4_DECODE_CASE)
#undef NVFP4_DECODE_CASE
  return hipErrorInvalidValue;
}

#undef NVFP4_DECODE_SHAPES

}  // namespace nvfp4
