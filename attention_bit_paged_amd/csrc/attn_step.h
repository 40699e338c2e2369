// One 32-token step of paged NVFP4 attention for one wave, shared by the decode and
// prefill kernels.
//
// Layout (gfx950 wave64, 16x16x32 fp16 MFMA; lane l = 16j + n):
//   * S^T = K Q^T: K rows (tokens) on M, query rows on N.  Two token tiles per step:
//     tile A row m is token 8*(m/4) + m%4 of the step, tile B row m is that token + 4.
//     The accumulator layout (lane (j, n) holds rows 4j..4j+3 of column n) then gives
//     lane (j, n) the scores of tokens 8j..8j+7 for query row n.
//   * O^T += V^T P^T: value dims on M, tokens on K, query rows on N.  Lane (j, n)'s
//     k-slots are tokens 8j..8j+7, the same tokens it holds scores for, so P needs no
//     lane exchange.  Lane (j, m) reads for those 8 tokens the m-th 1/16 slice of the
//     V row; nibble e of the slice is value dim m*DV/16 + e and feeds PV tile e.
//   * The K contraction runs over each lane's contiguous quarter row: k-step s takes
//     dword s of the quarter row; Q is laid out with the same (lane, slot) order.
// Page sources: [XQA] "Support NVFP4 KV cache decode on SM120" (packed K/V and scale
// factors streamed through a page table); [PF] "Re-enable split-KV for NVFP4 KV cache in
// prefill path" (K and V through independent strides).
#pragma once

#include "fp4_common.h"
#include "internal.h"

namespace nvfp4 {

// Softmax reference point moves only when a row's maximum exceeds it by this much
// (base-2 units); until then exp2(x - ref) <= 2^8 and the accumulators stay untouched.
constexpr float kRescaleSlack = 8.f;

// Storage format of the K/V pools a kernel reads: NVFP4 (packed e2m1 pairs plus one
// e4m3 scale byte per 16 elements) or FP8 (one e4m3 byte per element, no block scales;
// the per-tensor scale is applied outside the step like NVFP4's global scale).
enum KvFmt : int { kNvfp4 = 0, kFp8 = 1 };

template <int DK, int DV, int FMT = kNvfp4>
struct StepShape {
  static constexpr bool F8 = FMT == kFp8;
  static constexpr int NS = DK / 32;     // QK k-steps (eight elements of a quarter row each)
  static constexpr int KSTEP = F8 ? 8 : 4;         // K bytes per lane and k-step
  static constexpr int KB = NS * KSTEP;  // K bytes per lane per token
  static constexpr int KBW = KB / 4;
  static constexpr int KSF = F8 ? 0 : DK / 64;     // K scale bytes per lane per token
  static constexpr int KSFW = (KSF + 3) / 4 > 0 ? (KSF + 3) / 4 : 1;
  static constexpr int KPAIRS = (KSF + 1) / 2;
  static constexpr int VB = F8 ? DV / 16 : DV / 32;  // V bytes per lane per token
  static constexpr int VW = (VB + 3) / 4;
  static constexpr int NT = DV / 16;     // PV tiles
  static constexpr int VSFB = F8 ? 0 : (DV >= 512 ? 2 : 1);  // V scale bytes per lane per token
  static constexpr int QW = DK / 8;      // dwords of a lane's bf16 Q quarter-row
  static constexpr int RBK = F8 ? DK : DK / 2;     // bytes of one K row
  static constexpr int RBV = F8 ? DV : DV / 2;
  static constexpr int SBK = F8 ? 0 : DK / 16;     // scale bytes of one K row
  static constexpr int SBV = F8 ? 0 : DV / 16;
};

template <int DK, int DV, int FMT = kNvfp4>
struct StepRaw {
  using S = StepShape<DK, DV, FMT>;
  uint32_t ka[S::KBW], kb[S::KBW];
  uint32_t ksa[S::KSFW], ksb[S::KSFW];
  uint32_t vd[8][S::VW];
  uint32_t vs[8];
};

// Per-wave view of one request's K/V pools for one kv head.
//
// PAGE16 (page_size >= 16): the two 16-token halves of a step each lie inside one page,
// so a step needs two page-table entries (uniform, scalar loads); the ring kernels
// take their copy bases from this view.  Otherwise (page_size < 16) load() looks every
// token up on its own.
template <int DK, int DV, bool PAGE16, int FMT = kNvfp4>
struct PagedView {
  using S = StepShape<DK, DV, FMT>;
  const int32_t* pt_row;
  int page_shift, page_mask, num_pages;
  const uint8_t* kdat;
  const uint8_t* ksf;
  const uint8_t* vdat;
  const uint8_t* vsf;
  int64_t k_page, k_tok, ksf_page, ksf_tok, v_page, v_tok, vsf_page, vsf_tok;
  int j, n;
  uint32_t bad;
  int stream;  // the ring copies may take the non-temporal policy (AttnArgs::stream_kv)

  __device__ __forceinline__ void init(const AttnArgs& a, int b, int kvh, int lane) {
    j = lane >> 4;
    n = lane & 15;
    pt_row = a.page_table + (int64_t)b * a.pt_stride;
    page_shift = a.page_shift;
    page_mask = (1 << a.page_shift) - 1;
    num_pages = a.k.num_pages;
    kdat = a.k.data + (int64_t)kvh * a.k.s_head;
    ksf = a.k.sf + (int64_t)kvh * a.k.sf_head;
    vdat = a.v.data + (int64_t)kvh * a.v.s_head;
    vsf = a.v.sf + (int64_t)kvh * a.v.sf_head;
    k_page = a.k.s_page; k_tok = a.k.s_tok; ksf_page = a.k.sf_page; ksf_tok = a.k.sf_tok;
    v_page = a.v.s_page; v_tok = a.v.s_tok; vsf_page = a.v.sf_page; vsf_tok = a.v.sf_tok;
    bad = 0;
    stream = a.stream_kv;
  }

  // A page-table entry; one outside [0, num_pages) marks the view bad and reads page 0
  // instead, so no address is ever formed from it.
  __device__ __forceinline__ int page_of(int idx) {
    int pg = pt_row[idx];
    if ((unsigned)pg >= (unsigned)num_pages) {
      bad = 1;
      pg = 0;
    }
    return pg;
  }

  // The page-table entries of a step's tokens for this lane (page_size < 16): the K
  // tiles' two tokens and the eight value tokens.  Read a step ahead of the step's data
  // (load below), so that a data load never waits for its page-table load.
  struct Pages {
    int ka, kb, v[8];
  };
  __device__ __forceinline__ void lookup(Pages& p, int t0, int tlast) const {
    static_assert(!PAGE16, "page_size >= 16 streams through the LDS rings");
    const int ta = min(t0 + 8 * (n >> 2) + (n & 3), tlast);
    const int tb = min(t0 + 8 * (n >> 2) + (n & 3) + 4, tlast);
    p.ka = pt_row[ta >> page_shift];
    p.kb = pt_row[tb >> page_shift];
#pragma unroll
    for (int i = 0; i < 8; ++i) p.v[i] = pt_row[min(t0 + 8 * j + i, tlast) >> page_shift];
  }
  // Raw bytes of the step starting at token t0 from its looked-up pages.  Keys after
  // tlast are never used; their reads are clamped to tlast.  An entry outside
  // [0, num_pages) marks the view bad and reads page 0 instead.
  __device__ __forceinline__ void load(StepRaw<DK, DV, FMT>& r, const Pages& p, int t0, int tlast) {
    auto valid = [&](int pg) {
      if ((unsigned)pg >= (unsigned)num_pages) {
        bad = 1;
        return 0;
      }
      return pg;
    };
    const int ta = min(t0 + 8 * (n >> 2) + (n & 3), tlast);
    const int tb = min(t0 + 8 * (n >> 2) + (n & 3) + 4, tlast);
    const int pga = valid(p.ka), pgb = valid(p.kb);
    load_bytes<S::KB>(kdat + pga * k_page + (int64_t)(ta & page_mask) * k_tok + j * S::KB, r.ka);
    load_bytes<S::KB>(kdat + pgb * k_page + (int64_t)(tb & page_mask) * k_tok + j * S::KB, r.kb);
    if constexpr (!S::F8) {
      load_bytes<S::KSF>(ksf + pga * ksf_page + (int64_t)(ta & page_mask) * ksf_tok + j * S::KSF, r.ksa);
      load_bytes<S::KSF>(ksf + pgb * ksf_page + (int64_t)(tb & page_mask) * ksf_tok + j * S::KSF, r.ksb);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = min(t0 + 8 * j + i, tlast);
      const int pg = valid(p.v[i]);
      const int64_t sl = t & page_mask;
      load_bytes<S::VB>(vdat + pg * v_page + sl * v_tok + n * S::VB, r.vd[i]);
      if constexpr (!S::F8)
        load_bytes<S::VSFB>(vsf + pg * vsf_page + sl * vsf_tok + (n * DV / 16) / 16, &r.vs[i]);
    }
  }
  // Both at once (a step whose pages were not looked up ahead).
  __device__ __forceinline__ void load(StepRaw<DK, DV, FMT>& r, int t0, int tlast) {
    Pages p;
    lookup(p, t0, tlast);
    load(r, p, t0, tlast);
  }
};

// Q quarter-row of one query row as fp16 MFMA operands, prescaled by a power of two
// that puts the row's largest magnitude in [2^14, 2^15) (exact for bf16 inputs in
// fp16's range).  Returns the factor that undoes the prescale on the scores.
template <int DK>
__device__ __forceinline__ float load_q_operand(const uint16_t* qrow, bool valid, int j,
                                                f16x8 (&qf)[DK / 32]) {
  constexpr int QW = DK / 8;
  uint32_t qraw[QW];
  if (valid) {
    load_bytes<DK / 2>(reinterpret_cast<const uint8_t*>(qrow + j * (DK / 4)), qraw);
  } else {
#pragma unroll
    for (int i = 0; i < QW; ++i) qraw[i] = 0u;
  }
  // The largest magnitude, as the largest sign-cleared bf16 bit pattern: for finite
  // values the unsigned order of those patterns is the order of the magnitudes (a row
  // holding a NaN or an infinity gives non-finite scores whatever its scale).
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 mb = {0, 0};
#pragma unroll
  for (int i = 0; i < QW; ++i)
    mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, qraw[i] & 0x7FFF7FFFu));
  float qmax = __uint_as_float((uint32_t)(mb[0] > mb[1] ? mb[0] : mb[1]) << 16);
  qmax = max_over_groups(qmax);
  int qexp = 0;
  if (qmax > 0.f) (void)frexpf(qmax, &qexp);
  const float qmul = ldexpf(1.f, 15 - qexp);
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    f16x2 p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w = qraw[4 * s + t];
      p[t] = f16x2{(_Float16)(bf16f(w & 0xFFFF) * qmul), (_Float16)(bf16f(w >> 16) * qmul)};
    }
    qf[s] = pack8(p[0], p[1], p[2], p[3]);
  }
  return ldexpf(1.f, qexp - 15);
}

// Eight consecutive e4m3 bytes (two dwords, element 0 in the low byte) -> exact fp16.
__device__ __forceinline__ f16x8 fp8x8_to_f16(uint32_t w0, uint32_t w1) {
  return pack8(fp8x2_to_f16<false>(w0), fp8x2_to_f16<true>(w0), fp8x2_to_f16<false>(w1),
               fp8x2_to_f16<true>(w1));
}

// Dequantised K operands of the two token tiles of a step.
template <int DK, int DV, int FMT>
__device__ __forceinline__ void k_operands(const StepRaw<DK, DV, FMT>& r, f16x8 (&ka)[DK / 32],
                                           f16x8 (&kb)[DK / 32]) {
  using S = StepShape<DK, DV, FMT>;
  if constexpr (S::F8) {
#pragma unroll
    for (int s = 0; s < S::NS; ++s) {
      ka[s] = fp8x8_to_f16(r.ka[2 * s], r.ka[2 * s + 1]);
      kb[s] = fp8x8_to_f16(r.kb[2 * s], r.kb[2 * s + 1]);
    }
  } else {
  f16x2 kpa[S::KPAIRS], kpb[S::KPAIRS];
#pragma unroll
  for (int w = 0; w < S::KPAIRS; ++w) {
    kpa[w] = (w & 1) ? fp8x2_to_f16<true>(r.ksa[w >> 1]) : fp8x2_to_f16<false>(r.ksa[w >> 1]);
    kpb[w] = (w & 1) ? fp8x2_to_f16<true>(r.ksb[w >> 1]) : fp8x2_to_f16<false>(r.ksb[w >> 1]);
  }
#pragma unroll
  for (int s = 0; s < S::NS; ++s) {
    const int bi = s >> 1;  // scale byte of this dword within the lane's quarter-row
    const f16x2 sca = (bi & 1) ? splat_hi(kpa[bi >> 1]) : splat_lo(kpa[bi >> 1]);
    const f16x2 scb = (bi & 1) ? splat_hi(kpb[bi >> 1]) : splat_lo(kpb[bi >> 1]);
    ka[s] = dequant8(r.ka[s], sca);
    kb[s] = dequant8(r.kb[s], scb);
  }
}
}

// FP8: the byte transposition pairs the tokens of a k-slot pair: for dword q of the
// slices of tokens 2p and 2p+1, v_perm_b32 gathers element 4q+e of both tokens into
// one fp8 pair, which one convert turns into the fp16 pair of PV tile 4q+e.  Tokens
// after tlast (MASK) read as zero bytes.
template <int DK, int DV, bool MASK>
__device__ __forceinline__ void v_operands_fp8(const StepRaw<DK, DV, kFp8>& r, int t0, int tlast,
                                               int j, f16x8 (&vt)[DV / 16]) {
  using S = StepShape<DK, DV, kFp8>;
  f16x2 vp[S::NT][4];
#pragma unroll
  for (int q = 0; q < S::VW; ++q) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t w0 = r.vd[2 * p][q], w1 = r.vd[2 * p + 1][q];
      if constexpr (MASK) {
        if (t0 + 8 * j + 2 * p > tlast) w0 = 0u;
        if (t0 + 8 * j + 2 * p + 1 > tlast) w1 = 0u;
      }
      // bytes {w0.b0, w1.b0, w0.b1, w1.b1} and {w0.b2, w1.b2, w0.b3, w1.b3}
      const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
      const uint32_t hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
      vp[4 * q + 0][p] = fp8x2_to_f16<false>(lo);
      vp[4 * q + 1][p] = fp8x2_to_f16<true>(lo);
      vp[4 * q + 2][p] = fp8x2_to_f16<false>(hi);
      vp[4 * q + 3][p] = fp8x2_to_f16<true>(hi);
    }
  }
#pragma unroll
  for (int e = 0; e < S::NT; ++e) vt[e] = pack8(vp[e][0], vp[e][1], vp[e][2], vp[e][3]);
}

template <int DK, int DV, bool MASK, int FMT>
__device__ __forceinline__ void v_operands(const StepRaw<DK, DV, FMT>& r, int t0, int tlast, int j,
                                           f16x8 (&vt)[DV / 16]) {
  if constexpr (FMT == kFp8) {
    v_operands_fp8<DK, DV, MASK>(r, t0, tlast, j, vt);
    return;
  } else {
  using S = StepShape<DK, DV>;
  uint32_t sw[S::VSFB][2];
#pragma unroll
  for (int h = 0; h < S::VSFB; ++h) {
    uint32_t bytes[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bytes[i] = (r.vs[i] >> (8 * h)) & 0xFF;
      if constexpr (MASK) bytes[i] = (t0 + 8 * j + i > tlast) ? 0u : bytes[i];
    }
    sw[h][0] = bytes[0] | (bytes[1] << 8) | (bytes[2] << 16) | (bytes[3] << 24);
    sw[h][1] = bytes[4] | (bytes[5] << 8) | (bytes[6] << 16) | (bytes[7] << 24);
  }
  f16x2 vp[S::NT][4];
#pragma unroll
  for (int q = 0; q < S::VW; ++q) {
    const int h = (q * 8) / 16 < S::VSFB ? (q * 8) / 16 : 0;  // scale block of this dword
    const f16x2 sp[4] = {fp8x2_to_f16<false>(sw[h][0]), fp8x2_to_f16<true>(sw[h][0]),
                         fp8x2_to_f16<false>(sw[h][1]), fp8x2_to_f16<true>(sw[h][1])};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t w0 = r.vd[2 * p][q];
      const uint32_t w1 = r.vd[2 * p + 1][q];
      // byte k of lo: nibble 2k of token 2p (low) and of token 2p+1 (high); hi: nibble 2k+1
      const uint32_t lo = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);
      const uint32_t hi = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);
      constexpr int NB = S::VB < 4 ? S::VB : 4;  // bytes of the slice in this dword
      if constexpr (NB > 0) { vp[8 * q + 0][p] = fp4x2_to_f16<0>(lo) * sp[p]; vp[8 * q + 1][p] = fp4x2_to_f16<0>(hi) * sp[p]; }
      if constexpr (NB > 1) { vp[8 * q + 2][p] = fp4x2_to_f16<1>(lo) * sp[p]; vp[8 * q + 3][p] = fp4x2_to_f16<1>(hi) * sp[p]; }
      if constexpr (NB > 2) { vp[8 * q + 4][p] = fp4x2_to_f16<2>(lo) * sp[p]; vp[8 * q + 5][p] = fp4x2_to_f16<2>(hi) * sp[p]; }
      if constexpr (NB > 3) { vp[8 * q + 6][p] = fp4x2_to_f16<3>(lo) * sp[p]; vp[8 * q + 7][p] = fp4x2_to_f16<3>(hi) * sp[p]; }
    }
  }
#pragma unroll
  for (int e = 0; e < S::NT; ++e) vt[e] = pack8(vp[e][0], vp[e][1], vp[e][2], vp[e][3]);
  }
}

// Custom masks (packed bits, 1 = visible; element i*L + j of a request's [q, L] mask is
// bit (e % 8) of byte e / 8 of its segment).  The visibility of the lane's eight keys
// key0 .. key0 + 7 for query row `qpos`: only the first `nvalid` of them exist (the
// rest read as hidden), and only the bytes holding those bits are read.
__device__ __forceinline__ uint32_t mask_bits8(const uint8_t* seg, int64_t L, int qpos, int key0,
                                               int nvalid) {
  if (nvalid <= 0) return 0u;
  nvalid = nvalid > 8 ? 8 : nvalid;
  const int64_t bit = (int64_t)qpos * L + key0;
  const int sh = (int)(bit & 7);
  uint32_t w = seg[bit >> 3];
  if (sh + nvalid > 8) w |= (uint32_t)seg[(bit >> 3) + 1] << 8;
  return (w >> sh) & ((1u << nvalid) - 1u);
}

// Multiplies 16 accumulators by alpha in place.  One asm statement whose operands are
// the accumulators themselves: under a branch, the registers stay where they are (as
// C++ arithmetic, the join of the two paths copies every accumulator).  The leading
// nops cover the MFMA-result-to-VALU distance, the trailing ones the VALU-to-MFMA
// operand one.  Not volatile: the operands order it, and a volatile statement would
// end the scheduling region around it.
__device__ __forceinline__ void scale16(f32x4& a, f32x4& b, f32x4& c, f32x4& d, float alpha) {
  asm(
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
      "v_mul_f32 %0, %0, %16\n\tv_mul_f32 %1, %1, %16\n\tv_mul_f32 %2, %2, %16\n\t"
      "v_mul_f32 %3, %3, %16\n\tv_mul_f32 %4, %4, %16\n\tv_mul_f32 %5, %5, %16\n\t"
      "v_mul_f32 %6, %6, %16\n\tv_mul_f32 %7, %7, %16\n\tv_mul_f32 %8, %8, %16\n\t"
      "v_mul_f32 %9, %9, %16\n\tv_mul_f32 %10, %10, %16\n\tv_mul_f32 %11, %11, %16\n\t"
      "v_mul_f32 %12, %12, %16\n\tv_mul_f32 %13, %13, %16\n\tv_mul_f32 %14, %14, %16\n\t"
      "v_mul_f32 %15, %15, %16\n\ts_nop 4"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]),
        "+v"(b[3]), "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(d[0]), "+v"(d[1]),
        "+v"(d[2]), "+v"(d[3])
      : "v"(alpha));
}

// Where the accumulators of a RowState live: VGPRs rescaled in place by scale16, or
// left to plain code.
enum class AccForm { VGPR, PLAIN };

// Online-softmax state of one 16-row group (base-2 scores).  `m` is a reference point,
// not necessarily the running maximum: it is raised only when a row's maximum exceeds
// it by kRescaleSlack, so p = exp2(x - m) <= 2^8.  O = acc / l and LSE = m + log2(l)
// hold for any reference point; `l` is this lane's share of the row sum (its 8 keys of
// every step), completed over the row's four lanes at the end.  A step forms the
// row-wide maximum (a cross-lane exchange) only when some lane of the wave holds a key
// more than the slack above the reference, which is rare once the reference has
// settled; the other lanes of its row can only be lower.
template <int NT, AccForm FORM>
struct RowState {
  f32x4 acc[NT];
  float m, l;
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int e = 0; e < NT; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }

  // Scores of tokens t0 + 8j + i (i < 8) for this lane's row: sa (i < 4), sb (i >= 4).
  // With MASK, keys after `last` are dropped; without it every key is valid, so the
  // reference point is finite once this step has been folded in.  Returns the P operand.
  template <bool MASK>
  __device__ __forceinline__ f16x8 softmax(f32x4 sa, f32x4 sb, float c, int t0, int j, int last) {
    float x[8];
    const float bm = scores<MASK>(sa, sb, t0, j, last, x);
    if (__ballot(wants(bm, c)) != 0) raise(bm, c);
    return probs<MASK>(x, c);
  }

  // The softmax in parts, for callers that hold several row groups and keep the rare
  // rescale branch apart from the exponentials.  scores(): the step's raw scores x (c
  // times them is the base-2 exponent; c > 0, the host rejects other scales) with
  // masked keys at -inf, and this lane's largest.
  template <bool MASK>
  __device__ __forceinline__ float scores(f32x4 sa, f32x4 sb, int t0, int j, int last, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = sa[i];
      x[4 + i] = sb[i];
    }
    if constexpr (MASK) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (t0 + 8 * j + i > last) x[i] = -INFINITY;
    }
    // Compiler-generated code, not asm: the scores come straight from the matrix unit,
    // and only compiler-generated code gets the wait states a VALU read of an MFMA
    // result needs.  The NaN-propagating maximum (four v_maximum3_f32) rather than
    // fmaxf, whose IEEE semantics make the compiler quieten some MFMA results first; a
    // NaN score could only come from a key that is masked above or from NaN inputs.
    const float b1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]), x[2]);
    const float b2 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[3], x[4]), x[5]);
    const float b3 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[6], x[7]), b1);
    return __builtin_elementwise_maximum(b3, b2);
  }
  // The same with visibility given bit by bit (a custom mask): key t0 + 8j + i is
  // visible when bit i of `vis` is set.
  __device__ __forceinline__ float scores_vis(f32x4 sa, f32x4 sb, uint32_t vis, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = sa[i];
      x[4 + i] = sb[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!((vis >> i) & 1u)) x[i] = -INFINITY;
    const float b1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]), x[2]);
    const float b2 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[3], x[4]), x[5]);
    const float b3 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[6], x[7]), b1);
    return __builtin_elementwise_maximum(b3, b2);
  }
  __device__ __forceinline__ f16x8 softmax_vis(f32x4 sa, f32x4 sb, float c, uint32_t vis) {
    float x[8];
    const float bm = scores_vis(sa, sb, vis, x);
    if (__ballot(wants(bm, c)) != 0) raise(bm, c);
    return probs<true>(x, c);
  }
  // This lane's largest passes the reference by more than the slack.  bm * c - m is
  // +inf while m is -inf (any key raises) and NaN when both are -inf (the lane has no
  // key yet: nothing to raise).
  __device__ __forceinline__ bool wants(float bm, float c) const {
    return fmaf(bm, c, -m) > kRescaleSlack;
  }
  // Under a wave-uniform branch taken when some lane wants it: forms the row-wide
  // maximum and moves the reference of the rows that passed it by the slack.
  __device__ __forceinline__ void raise(float bm, float c) {
    const float bmr = max_over_groups(bm) * c;  // the row's largest scaled score
    const bool up = bmr > m + kRescaleSlack;
    const float m_new = up ? bmr : m;
    const float alpha = up ? fast_exp2(m - m_new) : 1.f;  // 0 when m was -inf
    if constexpr (FORM == AccForm::VGPR) {
#pragma unroll
      for (int e = 0; e < NT; e += 4) scale16(acc[e], acc[e + 1], acc[e + 2], acc[e + 3], alpha);
    } else {
#pragma unroll
      for (int e = 0; e < NT; ++e) acc[e] *= alpha;
    }
    l *= alpha;
    m = m_new;
  }
  // P = exp2(x c - m) in fp16, and the lane's row sum, which takes the fp16 values the
  // PV product uses.
  template <bool MASK>
  __device__ __forceinline__ f16x8 probs(const float (&x)[8], float c) {
    const float m_use = MASK ? (m == -INFINITY ? 0.f : m) : m;
    f16x2 pp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = fast_exp2(fmaf(x[2 * i], c, -m_use));
      const float p1 = fast_exp2(fmaf(x[2 * i + 1], c, -m_use));
      pp[i] = f16x2{(_Float16)p0, (_Float16)p1};
    }
    const f16x2 one2 = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) l = __builtin_amdgcn_fdot2(pp[i], one2, l, false);
    return pack8(pp[0], pp[1], pp[2], pp[3]);
  }

  __device__ __forceinline__ void pv(const f16x8 (&vt)[NT], f16x8 p) {
#pragma unroll
    for (int e = 0; e < NT; ++e) acc[e] = mfma16x16x32(vt[e], p, acc[e]);
  }

  // A split work item's partial state: this lane's part of the row normalised by its own
  // row sum, in fp16 (the layout of store), and its LSE.  The global V scale is left to
  // the merge, so the values stay within fp16's range: a normalised row is a convex
  // combination of dequantised values (|v| <= 6 x 448).  Each value is rounded once, a
  // relative error of at most 2^-11.
  __device__ __forceinline__ void store_partial(_Float16* dst, float* lse_dst, bool valid, bool bad,
                                                int j) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const float l_tot = sum_over_groups(l);
    const bool empty = !(l_tot > 0.f);
    const float inv = bad ? NAN : (empty ? 0.f : 1.f / l_tot);
    const float lse_v =
        bad ? NAN : (empty ? -INFINITY : (m + fast_log2(l_tot)) * 0.69314718055994531f);
    if (!valid) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x4* row = reinterpret_cast<f16x4*>(dst + (4 * j + i) * NT);
#pragma unroll
      for (int e = 0; e < NT; e += 4)
        row[e / 4] = f16x4{(_Float16)(acc[e][i] * inv), (_Float16)(acc[e + 1][i] * inv),
                           (_Float16)(acc[e + 2][i] * inv), (_Float16)(acc[e + 3][i] * inv)};
    }
    if (j == 0) *lse_dst = lse_v;
  }

  // Normalise and store this lane's part of the row: value dims (4j+i)*NT + e.  The row
  // sum is first completed over the four lanes of the row.
  __device__ __forceinline__ void store(float* dst, float* lse_dst, bool valid, bool bad,
                                        float out_scale, int j) {
    const float l_tot = sum_over_groups(l);
    const bool empty = !(l_tot > 0.f);
    const float inv = bad ? NAN : (empty ? 0.f : out_scale / l_tot);
    const float lse_v =
        bad ? NAN : (empty ? -INFINITY : (m + fast_log2(l_tot)) * 0.69314718055994531f);
    if (!valid) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4* row = reinterpret_cast<float4*>(dst + (4 * j + i) * NT);
#pragma unroll
      for (int e = 0; e < NT; e += 4)
        row[e / 4] = make_float4(acc[e][i] * inv, acc[e + 1][i] * inv, acc[e + 2][i] * inv,
                                 acc[e + 3][i] * inv);
    }
    if (j == 0) *lse_dst = lse_v;
  }
};

}  // namespace nvfp4
