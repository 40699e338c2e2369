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
// major, so the heads that share a kv head share every K/V byte read.
//
// Cooperative kernel: the workgroup streams the chunk in 32-token steps.  The raw
// packed bytes of a step arrive in a shared LDS ring by direct global-to-LDS copies
// (each wave issues one pool's copies, three steps deep); the four waves then
// dequantise the step together into fp16 MFMA operands, stored lane-major in an LDS
// operand buffer (double-buffered, one barrier per step), and every wave computes its
// groups of 16 rows from those operands, held in registers for the step (three groups
// per wave for head dims up to 128).  The K/V dequantisation and the LDS reads are thus
// shared by all rows of the tile.  Pages of 16 tokens or more give each copy a base per
// 16-token half; smaller pages (SMALL) give each copy lane its own address, from the
// step's page-table entries that stream into LDS with the copies.
//
// A split tile's partial states are merged by a separate kernel.
#pragma once

#include <type_traits>

#include "kv_ring.h"
#include "rope.h"

namespace nvfp4 {

namespace {

// Operand registers of the wide-head (DK = 512) cooperative kernel's LDS read pipeline:
// reads run this many k-steps (V tiles) less one ahead of their products (3 and 5
// measured alike, 7 slower).
constexpr int kWidePrefetch = 3;
// Row groups of 16 per wave of the wide-head kernel (waves: 8 / groups).  Two groups
// (four waves, one per SIMD, half the operand reads per product) measured 8 % slower:
// with one wave per SIMD the LDS and barrier latencies are exposed.
constexpr int kWideGroups = 1;

// ------------------------------------------------------------------ cooperative --

template <int DK, int DV, int FMT = kNvfp4>
struct CoopShape {
  using S = StepShape<DK, DV, FMT>;
  static constexpr bool OK = (DK <= 256 && DV <= 256) || (DK == 512 && DV <= 256);
  // Head dims up to 128: four waves of three row groups, two workgroups per CU (two
  // waves per SIMD hide each other's latencies, and the two workgroups' barriers are
  // independent); up to 256: four waves of two row groups, one wave per SIMD.
  static constexpr bool SMALL = DK <= 128 && DV <= 128;
  // DK = 512: the K operands of a step (a quarter of the register file) are read one
  // k-step at a time and the V operands one tile at a time; eight waves of one row
  // group each, two per SIMD, so that one wave's LDS reads overlap the other's products.
  static constexpr bool WIDE = DK > 256;
  static constexpr int NW = WIDE ? 8 / kWideGroups : 4;
  static constexpr int NR = SMALL ? 3 : (WIDE ? kWideGroups : 2);  // row groups of 16 per wave
  static constexpr int WGS_PER_CU = SMALL ? 2 : 1;
  static constexpr int ROWS = NW * NR * 16;       // rows per work item
  static constexpr int NOP = 2 * S::NS + S::NT;   // operand vectors per step
  static constexpr int OPB = NOP * 64 * 16;       // bytes of one operand buffer
  static constexpr int RAW_STAGE = RingBytes<DK, DV, FMT>::STAGE;  // a step's K/V bytes
  static constexpr int WL = 3 * RAW_STAGE;
  using R = RingShape<DK, DV, WL, FMT>;           // three raw stages
  // A step's custom-mask bytes: 8 per tile query (two 4-byte copies of 64 lanes per
  // block of 64 queries; a tile has at most ROWS queries), in a ring of four slots of
  // their own: the copies of step s land in slot s % 4 three steps ahead, and that slot
  // is written again only after step s's softmax, so the step reads its bits directly.
  static constexpr int MASK_BLOCKS = (ROWS + 63) / 64;
  static constexpr int MASK_SLOT = MASK_BLOCKS * 512;
  static constexpr int LDS = 3 * RAW_STAGE + 2 * OPB;  // without the mask ring
  static constexpr int LDS_MASKED = LDS + 4 * MASK_SLOT;
  static constexpr int ROPE_TAB = DK * 4;          // RoPE: DK/2 frequency pairs of floats
  static constexpr int LDS_ROPE = LDS + ROPE_TAB;
  static constexpr int KE = (2 * S::NS + NW - 1) / NW;  // K operand entries per lane
  // 512-dim heads (without RoPE): a lane dequantises one 16-byte piece of a key row into
  // four K entries (see CoopLanes); the ring holds each key row's pieces rotated
  static constexpr bool piece(bool rope) { return WIDE && !rope && FMT == kNvfp4; }
  static constexpr int VH = NW / 4;               // V tiles split in this many parts
  static constexpr int VPART = S::NT / VH;        // V tiles per part
  static_assert(R::NST == 3, "raw ring depth");
  static_assert(S::NT % VH == 0, "V split");
};

constexpr int kLdsPerCu = 160 * 1024;

// LDS of one cooperative workgroup: three raw stages of 32 tokens (rows and, for NVFP4,
// scale rows) and two fp16 operand buffers (2 NS K entries and NT V tiles of 64 lanes x
// 16 bytes).  A formula, so that shapes without a kernel can be priced too.
// SMALL (pages below 16 tokens): four copy roles' page-table entry slots (4 x 256 bytes each).
constexpr int kCoopEntryBytes = 4 * 4 * 256;
constexpr int coop_lds_formula(int dk, int dv, int fmt, bool masked, bool rope = false,
                               bool small = false) {
  const int rbk = fmt == kFp8 ? dk : dk / 2, rbv = fmt == kFp8 ? dv : dv / 2;
  const int sf = fmt == kFp8 ? 0 : (2 * dk + 2 * dv + 255) / 256 * 256;
  const int rows = dk <= 128 && dv <= 128 ? 192 : 128;  // tile rows (queries at most)
  const int raw = 32 * (rbk + rbv) + sf;
  const int opb = (2 * (dk / 32) + dv / 16) * 64 * 16;
  return 3 * raw + 2 * opb + (masked ? 4 * ((rows + 63) / 64 * 512) : 0) + (rope ? 4 * dk : 0) +
         (small ? kCoopEntryBytes : 0);
}
constexpr int coop_wgs_per_cu(int dk, int dv) { return dk <= 128 && dv <= 128 ? 2 : 1; }

// Per-lane LDS offsets of the cooperative dequantisation (constant for the kernel).
// Operand o < 2*NS is K tile o/NS (token tile A or B), k-step o%NS; operand 2*NS + e is
// V^T tile e.  Entry (o, lane) is the 16 bytes lane `lane` loads for operand o.  K
// entries: wave w makes entries (w + NW*r, lane).  V: lane L of the workgroup makes,
// for the operand lane c = L / (4*VH), the token pair p = L%4 of the V tiles of part
// (L/4)%VH.
template <int DK, int DV, int FMT = kNvfp4, bool ROPE = false>
struct CoopLanes {
  using S = StepShape<DK, DV, FMT>;
  using C = CoopShape<DK, DV, FMT>;
  using R = typename C::R;
  // RoPE: the two lanes that hold partner elements of a key row (head-dim indices i and
  // i + DK/2: lane groups j and j + 2 of an entry) are made by one lane, so that each
  // angle is formed once per workgroup.  Lane (j, n) makes, for each pair q < KJ, both
  // halves of entry 2q + (j >> 1) of its wave: its lanes (j & 1, n) and ((j & 1) + 2, n).
  // Entry 2q + h then lies a fixed distance from entry h (NW divides NS / 2, or a wave
  // has at most two entries); the lanes of a missing entry (one entry per wave) make
  // nothing.
  static constexpr int KJ = ROPE ? (C::KE + 1) / 2 : C::KE;
  static_assert(!ROPE || C::KE <= 2 || S::NS % (2 * C::NW) == 0, "RoPE pair spacing");
  static constexpr int tok_off(int q) { return 4 * ((C::NW * 2 * q) / S::NS); }
  static constexpr uint32_t tab_off(int q) { return 64 * ((C::NW * 2 * q) % S::NS); }
  // Entry r of a lane is operand wave + NW*r.  NW divides NS (or a lane has one entry),
  // so entry r lies a fixed distance from entry 0 in the raw stage and in the operand
  // buffer: one per-lane base per pool, the rest immediate offsets of the LDS accesses.
  static_assert(S::NS % C::NW == 0 || C::KE == 1, "K entry spacing");
  static constexpr uint32_t k_raw_off(int r) {
    return (C::NW * r) / S::NS * 4 * S::RBK + S::KSTEP * ((C::NW * r) % S::NS);
  }
  static constexpr uint32_t k_sc_off(int r) {
    return (C::NW * r) / S::NS * 4 * S::SBK + ((C::NW * r) % S::NS) / 2;
  }
  static constexpr uint32_t k_dst_off(int r) { return C::NW * r * 64 * 16; }
  uint32_t k_raw, k_sc, k_dst;  // entry 0 (RoPE: the first half of the lane's entry of pair 0)
  uint32_t v_raw, v_sc, v_dst;
  int v_tok, part;
  int k_tok;       // RoPE: token (within the step) of the lane's entry of pair 0
  uint32_t k_tab;  // RoPE: LDS address of that entry's first frequency pair
  bool k_live;     // RoPE: the lane's entry exists

  // `tab`: LDS address of the RoPE frequency table (unused otherwise)
  __device__ __forceinline__ void init(int wave, int lane, uint32_t tab = 0) {
    const int j = lane >> 4, n = lane & 15;
    if constexpr (ROPE) {
      const int h = j >> 1, jj = j & 1;
      k_live = h < C::KE;
      const int o = min(wave + C::NW * h, 2 * S::NS - 1);
      const int tile = o / S::NS, s = o % S::NS;
      k_tok = 8 * (n >> 2) + (n & 3) + 4 * tile;
      k_raw = R::OFF_KD + k_tok * S::RBK + jj * S::KB + S::KSTEP * s;
      k_sc = R::OFF_SF + k_tok * S::SBK + jj * S::KSF + (s >> 1);
      k_dst = (o * 64 + 16 * jj + n) * 16;
      k_tab = tab + 8 * (jj * (DK / 4) + 8 * s);
    } else if constexpr (C::piece(ROPE)) {
      // Wave w covers k-steps 4(w%4)..4(w%4)+3 of token tile w/4; lane (j, n) reads the
      // 16-byte piece 4j + w%4 of its token's row (the lane's dwords of those four
      // k-steps) and its two scale bytes, and writes entry (j, n) of the four operands.
      // Key row t's piece p sits in LDS slot (p + n) % 16 of the row (n: the token's
      // column), so that each quarter-wave's 16 reads cover all banks.
      static_assert(S::NS == 16 && S::RBK == 256 && C::NW == 8, "piece layout");
      const int tile = wave >> 2, g = wave & 3, p = 4 * j + g;
      k_tok = 8 * (n >> 2) + (n & 3) + 4 * tile;
      k_raw = R::OFF_KD + k_tok * S::RBK + 16 * ((p + n) & 15);
      k_sc = R::OFF_SF + k_tok * S::SBK + 2 * p;
      k_dst = ((tile * S::NS + 4 * g) * 64 + lane) * 16;
      k_tab = 0;
      k_live = true;
    } else {
      const int o = min(wave, 2 * S::NS - 1);  // clamped: unused when past the end
      const int tile = o / S::NS, s = o % S::NS;
      k_tok = 8 * (n >> 2) + (n & 3) + 4 * tile;
      k_raw = R::OFF_KD + k_tok * S::RBK + j * S::KB + S::KSTEP * s;
      k_sc = R::OFF_SF + k_tok * S::SBK + j * S::KSF + (s >> 1);
      k_dst = (o * 64 + lane) * 16;
      k_tab = 0;
      k_live = true;
    }
    const int L = wave * 64 + lane;
    const int c = L / (4 * C::VH), p = L & 3;
    part = (L >> 2) % C::VH;
    const int jj = c >> 4, m = c & 15;
    v_tok = 8 * jj + 2 * p;
    v_raw = R::OFF_VD + v_tok * S::RBV + m * S::VB;
    v_sc = R::OFF_SF + R::KS + v_tok * S::SBV + (m * (DV / 16)) / 16;
    v_dst = (2 * S::NS * 64 + c) * 16 + 4 * p;
  }
};

// The cooperative dequantisation of one raw stage: load() reads this lane's raw bytes
// and scales, store() writes its fp16 operand entries.  MASK: value rows past `kleft`
// (tokens of the step after the chunk's last key) get scale 0, so that their bytes,
// whatever they hold (NaN scales included), dequantise to finite zeros: a NaN there
// would reach every output through its zero probability.  Key rows past the end are
// left as they are: a bad key row only spoils its own scores, which the softmax of a
// step that holds such keys replaces by -inf.
template <int DK, int DV, int FMT = kNvfp4, bool ROPE = false>
struct CoopRaw {
  using S = StepShape<DK, DV, FMT>;
  using C = CoopShape<DK, DV, FMT>;
  using L = CoopLanes<DK, DV, FMT, ROPE>;
  static constexpr int NB = S::VB < 4 ? S::VB : 4;   // bytes of the V slice per dword
  static constexpr int EPD = S::F8 ? NB : 2 * NB;    // V tiles per slice dword
  static constexpr int KW = S::KSTEP / 4;            // dwords of one K entry
  static constexpr bool PIECE = C::piece(ROPE);
  // RoPE: both halves of each pair; pieces: the piece's four dwords in kw[0]
  static constexpr int KSLOT = ROPE ? 2 * L::KJ : (PIECE ? 1 : C::KE);
  static constexpr int KWP = PIECE ? 4 : KW;
  uint32_t kw[KSLOT][KWP], ksc[KSLOT], sa, sb, vw0[S::VW], vw1[S::VW];

  __device__ __forceinline__ void load(uint32_t raw, int wave, const L& cl) {
    if constexpr (PIECE) {
      lds_load<16>(raw + cl.k_raw, kw[0]);
      lds_load<2>(raw + cl.k_sc, &ksc[0]);
    }
    if constexpr (ROPE) {
      // both halves of each of the lane's entries (its address clamped in range when
      // the entry does not exist)
#pragma unroll
      for (int q = 0; q < L::KJ; ++q) {
        const uint32_t at = raw + cl.k_raw + cl.k_raw_off(2 * q);
        lds_load<S::KSTEP>(at, kw[2 * q]);
        lds_load<S::KSTEP>(at + 2 * S::KB, kw[2 * q + 1]);
        if constexpr (!S::F8) {
          const uint32_t sc = raw + cl.k_sc + cl.k_sc_off(2 * q);
          lds_load<1>(sc, &ksc[2 * q]);
          lds_load<1>(sc + 2 * S::KSF, &ksc[2 * q + 1]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < (ROPE || PIECE ? 0 : C::KE); ++r) {
      // wave-uniform; always true when the K entries divide evenly among the waves
      if ((2 * S::NS) % C::NW == 0 || wave + C::NW * r < 2 * S::NS) {
        lds_load<S::KSTEP>(raw + cl.k_raw + cl.k_raw_off(r), kw[r]);
        if constexpr (!S::F8) lds_load<1>(raw + cl.k_sc + cl.k_sc_off(r), &ksc[r]);
      }
    }
    if constexpr (!S::F8) {
      const uint32_t vs = raw + cl.v_sc;
      lds_load<1>(vs, &sa);
      lds_load<1>(vs + DV / 16, &sb);
    }
    const uint32_t vr = raw + cl.v_raw;
#pragma unroll
    for (int q = 0; q < S::VW; ++q) {
      if (C::VH > 1 && C::VPART >= EPD && (q * EPD) / C::VPART != cl.part) continue;
      lds_load<NB>(vr + 4 * q, &vw0[q]);
      lds_load<NB>(vr + S::RBV + 4 * q, &vw1[q]);
    }
  }
  // `tpos`: position of the step's first key (RoPE)
  template <bool MASK>
  __device__ __forceinline__ void store(uint32_t opb, int wave, const L& cl, int kleft,
                                        float tpos);
};

template <int DK, int DV, int FMT, bool ROPE>
template <bool MASK>
__device__ __forceinline__ void CoopRaw<DK, DV, FMT, ROPE>::store(uint32_t opb, int wave,
                                                                  const L& cl, int kleft,
                                                                  float tpos) {
  typedef __attribute__((address_space(3))) uint8_t* lds_p;
  if constexpr (ROPE) {
#pragma unroll
    for (int q = 0; q < L::KJ; ++q) {
      f16x8 lo, hi;
      if constexpr (S::F8) {
        lo = fp8x8_to_f16(kw[2 * q][0], kw[2 * q][1]);
        hi = fp8x8_to_f16(kw[2 * q + 1][0], kw[2 * q + 1][1]);
      } else {
        lo = dequant8(kw[2 * q][0], splat_lo(fp8x2_to_f16<false>(ksc[2 * q])));
        hi = dequant8(kw[2 * q + 1][0], splat_lo(fp8x2_to_f16<false>(ksc[2 * q + 1])));
      }
      rope_k_pair(lo, hi, tpos + (float)(cl.k_tok + L::tok_off(q)), cl.k_tab + L::tab_off(q));
      // wave-uniform but for the one-entry case
      if (C::KE % 2 == 0 || q + 1 < L::KJ || cl.k_live) {
        const uint32_t at = opb + cl.k_dst + cl.k_dst_off(2 * q);
        *(__attribute__((address_space(3))) f16x8*)(lds_p)(size_t)at = lo;
        *(__attribute__((address_space(3))) f16x8*)(lds_p)(size_t)(at + 32 * 16) = hi;
      }
    }
  }
  if constexpr (PIECE) {
    // dword q of the piece is k-step 4(w%4) + q; the two scales cover dwords 0-1 and 2-3
    const f16x2 sc2 = fp8x2_to_f16<false>(ksc[0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f16x8 v = dequant8(kw[0][q], q < 2 ? splat_lo(sc2) : splat_hi(sc2));
      *(__attribute__((address_space(3))) f16x8*)(lds_p)(size_t)(opb + cl.k_dst + q * 1024) = v;
    }
  }
#pragma unroll
  for (int r = 0; r < (ROPE || PIECE ? 0 : C::KE); ++r) {
    if ((2 * S::NS) % C::NW == 0 || wave + C::NW * r < 2 * S::NS) {
      f16x8 v;
      if constexpr (S::F8)
        v = fp8x8_to_f16(kw[r][0], kw[r][1]);
      else
        v = dequant8(kw[r][0], splat_lo(fp8x2_to_f16<false>(ksc[r])));
      *(__attribute__((address_space(3))) f16x8*)(lds_p)(size_t)(opb + cl.k_dst + cl.k_dst_off(r)) = v;
    }
  }
  const uint32_t vd = opb + cl.v_dst;
  if constexpr (S::F8) {
    // value rows past the chunk's last key read as zero bytes; the byte transposition
    // pairs tokens v_tok and v_tok + 1 for each element (see v_operands_fp8)
#pragma unroll
    for (int q = 0; q < S::VW; ++q) {
      if (C::VH > 1 && C::VPART >= EPD && (q * EPD) / C::VPART != cl.part) continue;
      const uint32_t w0 = MASK && cl.v_tok > kleft ? 0u : vw0[q];
      const uint32_t w1 = MASK && cl.v_tok + 1 > kleft ? 0u : vw1[q];
      const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
      const uint32_t hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
#pragma unroll
      for (int k = 0; k < EPD; ++k) {
        if (C::VH > 1 && C::VPART < EPD && k / C::VPART != cl.part) continue;
        const f16x2 v = k == 0 ? fp8x2_to_f16<false>(lo)
                               : (k == 1 ? fp8x2_to_f16<true>(lo)
                                         : (k == 2 ? fp8x2_to_f16<false>(hi) : fp8x2_to_f16<true>(hi)));
        *(__attribute__((address_space(3))) uint32_t*)(lds_p)(size_t)(vd + (EPD * q + k) * 1024) =
            f16x2_bits(v);
      }
    }
    return;
  } else {
  if (MASK && cl.v_tok > kleft) sa = 0;
  if (MASK && cl.v_tok + 1 > kleft) sb = 0;
  const f16x2 sp = fp8x2_to_f16<false>(sa | (sb << 8));
#pragma unroll
  for (int q = 0; q < S::VW; ++q) {
    // a part covers VPART consecutive tiles: whole dwords, or a share of one
    if (C::VH > 1 && C::VPART >= EPD && (q * EPD) / C::VPART != cl.part) continue;
    const uint32_t w0 = vw0[q], w1 = vw1[q];
    // byte k of lo: nibble 2k of token ta (low) and of token ta+1 (high); hi: nibble 2k+1
    const uint32_t lo = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);
    const uint32_t hi = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);
#pragma unroll
    for (int k = 0; k < EPD; ++k) {
      const int e = EPD * q + k;
      if (C::VH > 1 && C::VPART < EPD && k / C::VPART != cl.part) continue;
      const uint32_t src = (k & 1) ? hi : lo;
      f16x2 v;
      switch (k >> 1) {
        case 0: v = fp4x2_to_f16<0>(src); break;
        case 1: v = fp4x2_to_f16<1>(src); break;
        case 2: v = fp4x2_to_f16<2>(src); break;
        default: v = fp4x2_to_f16<3>(src); break;
      }
      v = v * sp;
      *(__attribute__((address_space(3))) uint32_t*)(lds_p)(size_t)(vd + e * 1024) = f16x2_bits(v);
    }
  }
  }
}

// Dequantises the raw stage at `raw` into the operand buffer at `opb`.  MASK: value rows
// past `kleft` get scale 0.  Every raw read first: the operand stores may not move above
// them (the compiler cannot tell the raw stage from the operand buffer).
template <int DK, int DV, bool MASK, int FMT, bool ROPE>
__device__ __forceinline__ void coop_dequant(uint32_t raw, uint32_t opb, int wave,
                                             const CoopLanes<DK, DV, FMT, ROPE>& cl, int kleft,
                                             float tpos) {
  CoopRaw<DK, DV, FMT, ROPE> r;
  r.load(raw, wave, cl);
  r.template store<MASK>(opb, wave, cl, kleft, tpos);
}

// Waits until this wave's copies of all but the newest issued step are done (or all
// of them).  Waves 0..3 each copy one pool; the others copy nothing.
// Wave 3 also copies the custom-mask bytes, two copies per block of 64 tile queries:
// `mask_copies` of them per step (0, 2, 4 or 6; wave-uniform).
// SMALL: roles 0, 1 and 2 copy the K rows, the V rows and every scale row (R::N_KD,
// R::N_VD and R::N_SF copies, each whole) plus one entry copy a step; role 3 copies only
// the mask bytes.
template <int DK, int DV, int FMT, bool SMALL = false>
__device__ __forceinline__ void coop_wait(int wave, bool one_newer, int mask_copies) {
  using R = typename CoopShape<DK, DV, FMT>::R;
  constexpr bool F8 = StepShape<DK, DV, FMT>::F8;
  constexpr int N0 = SMALL ? R::N_KD + 1 : R::ndma(1);
  constexpr int N1 = SMALL ? R::N_VD + 1 : R::ndma(2);
  constexpr int N2 = SMALL ? (F8 ? 0 : R::N_SF + 1) : R::ndma(4);
  constexpr int N3 = SMALL ? 0 : R::ndma(8);
  if (wave > 3) return;
  if (!one_newer) {
    asm volatile("s_waitcnt vmcnt(0)");
  } else if (wave == 0) {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N0));
  } else if (wave == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N1));
  } else if (wave == 2) {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N2));
  } else if (mask_copies == 0) {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N3));
  } else if (mask_copies == 2) {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N3 + 2));
  } else if (mask_copies == 4) {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N3 + 4));
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N3 + 6));
  }
}

// The custom-mask copies of a tile: lane l of block qb carries tile query 64 qb + l.
// A query's bits of the keys of a step start at byte ((q0 + l') L + t0) / 8 of the
// segment (t0 a multiple of 32), at a fixed bit shift; lanes past the tile's queries
// copy the tile's first query's bytes instead (unused).  The per-lane offsets are formed
// at each issue from scalars: held for the whole loop they were spilled, and a reload
// there waits for every copy in flight.
struct CoopMask {
  const uint8_t* seg;  // the request's mask segment
  int64_t q0, kv_len;  // the tile's first query (within the request), the request's keys
  int qn;              // the tile's queries
  int blocks;          // blocks of 64 tile queries (uniform)
  uint32_t ring;       // LDS address of the mask ring (uniform)
};

// The copy offsets of the one pool this wave issues (wave 0: K data, 1: V data, 2 and 3:
// the scale bytes, whose copies carry both pools' lanes).  The full plan holds every
// pool's offsets; kept whole in each wave they cost registers the loop needs.
// RECOMPUTE (FP8 rows at two workgroups per CU, four offsets a wave): the offsets are
// formed from the lane at each issue instead; held for the loop they were spilled, and
// the reload before its copy waited for every copy in flight.
template <int DK, int DV, int FMT = kNvfp4>
struct CoopCopies {
  using R = RingShape<DK, DV, CoopShape<DK, DV, FMT>::WL, FMT>;
  using Plan = RingPlan<DK, DV, CoopShape<DK, DV, FMT>::WL, FMT>;
  static constexpr int MAXC = R::N_KD > R::N_VD ? (R::N_KD > R::N_SF ? R::N_KD : R::N_SF)
                                                : (R::N_VD > R::N_SF ? R::N_VD : R::N_SF);
  static constexpr bool RECOMPUTE = FMT == kFp8 && CoopShape<DK, DV, FMT>::WGS_PER_CU == 2;
  uint32_t mine[MAXC > 0 ? MAXC : 1];

  // Pieces: the K copies place piece p of step token t in slot (p + n(t)) % 16 of its
  // row, n(t) the token's column in its 16-token tile; so the copy lane that lands in
  // slot q fetches piece (q - n(t)) % 16.  Only the offset inside the row changes.
  template <class P>
  __device__ __forceinline__ static void rotate_k(P& rp, int lane) {
    static_assert(R::RBK == 256, "rotation of 16-piece rows");
#pragma unroll
    for (int c = 0; c < R::N_KD; ++c) {
      const int byte = c * 1024 + lane * 16;
      const int t = byte / R::RBK, q = (byte % R::RBK) / 16;
      const int nt = ((t >> 3) << 2) | (t & 3);
      rp.off[c] = rp.off[c] - (uint32_t)(16 * q) + (uint32_t)(16 * ((q - nt) & 15));
    }
  }
  __device__ __forceinline__ void init(const Plan& rp, int wave) {
    if constexpr (RECOMPUTE) return;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const uint32_t kd = c < R::N_KD ? rp.off[c] : 0u;
      const uint32_t vd = c < R::N_VD ? rp.off[R::N_KD + c] : 0u;
      const uint32_t sf = c < R::N_SF ? rp.off[R::N_KD + R::N_VD + c] : 0u;
      mine[c] = wave == 0 ? kd : (wave == 1 ? vd : sf);
    }
  }
  // a plan holding this wave's offsets in the places of pool P (1, 2, 4 or 8) and zeros
  // (never read for P) elsewhere
  template <int P>
  __device__ __forceinline__ Plan expand() const {
    Plan r;
    constexpr int first = P == 1 ? 0 : (P == 2 ? R::N_KD : R::N_KD + R::N_VD);
    constexpr int count = P == 1 ? R::N_KD : (P == 2 ? R::N_VD : R::N_SF);
#pragma unroll
    for (int c = 0; c < R::NCOPY; ++c)
      r.off[c] = (c >= first && c < first + count) ? mine[c - first] : 0u;
    return r;
  }
};

// SMALL: this role's copies of the step at t0 take their pages from the entry slot of
// that step (slots at `ids`, four of 256 bytes, the step's index mod 4), and the entry
// copy of the step three later goes out with them (see coop_wait).
template <int DK, int DV, int FMT, bool CMASK, bool SMALL = false, bool PIECE = false>
__device__ __forceinline__ void coop_issue(int wave, const CoopCopies<DK, DV, FMT>& cc,
                                           uint32_t stage, const PagedView<DK, DV, true, FMT>& view,
                                           int t0, int tlast, uint32_t& bad, const CoopMask& cm,
                                           int kv0, uint32_t ids = 0) {
  using C = CoopShape<DK, DV, FMT>;
  constexpr int WL = C::WL;
  if constexpr (SMALL) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));  // the offsets are formed here, at each issue
    SmallPlan<DK, DV, WL, FMT> sp;
    sp.init(lane, view);
    if constexpr (PIECE) CoopCopies<DK, DV, FMT>::rotate_k(sp, lane);
    const int m = (t0 - kv0) / kDecodeStep;
    const uint32_t slot = ids + (uint32_t)(m & 3) * 256, next = ids + (uint32_t)((m + 3) & 3) * 256;
    auto entries = [&]() {
      small_entries(next, view.pt_row, t0 + 3 * kDecodeStep, tlast, view.page_shift, lane);
    };
    if (wave == 0) {
      ring_issue_small<DK, DV, WL, 1, FMT>(sp, stage, slot, view, lane, bad);
      entries();
    } else if (wave == 1) {
      ring_issue_small<DK, DV, WL, 2, FMT>(sp, stage, slot, view, lane, bad);
      entries();
    } else if constexpr (!StepShape<DK, DV, FMT>::F8) {
      if (wave == 2) {
        ring_issue_small<DK, DV, WL, 0xC, FMT>(sp, stage, slot, view, lane, bad);
        entries();
      }
    }
  } else if constexpr (CoopCopies<DK, DV, FMT>::RECOMPUTE) {
    static_assert(StepShape<DK, DV, FMT>::F8, "FP8 only: no scale pools");
    // opaque at each issue, so that the offsets are formed here (see CoopCopies)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    typename CoopCopies<DK, DV, FMT>::Plan rp;
    rp.init(lane, view.k_tok, view.v_tok, view.ksf_tok, view.vsf_tok);
    if (wave == 0) ring_issue<DK, DV, WL, 1>(rp, stage, view, t0, tlast, bad);
    else if (wave == 1) ring_issue<DK, DV, WL, 2>(rp, stage, view, t0, tlast, bad);
  } else {
    if (wave == 0) ring_issue<DK, DV, WL, 1>(cc.template expand<1>(), stage, view, t0, tlast, bad);
    else if (wave == 1) ring_issue<DK, DV, WL, 2>(cc.template expand<2>(), stage, view, t0, tlast, bad);
    else if constexpr (!StepShape<DK, DV, FMT>::F8) {  // FP8 has no scale pools
      if (wave == 2) ring_issue<DK, DV, WL, 4>(cc.template expand<4>(), stage, view, t0, tlast, bad);
      else if (wave == 3) ring_issue<DK, DV, WL, 8>(cc.template expand<8>(), stage, view, t0, tlast, bad);
    }
  }
  if (CMASK && wave == 3) {
    const uint32_t slot = cm.ring + (((t0 - kv0) >> 5) & 3) * C::MASK_SLOT;
    int lane = threadIdx.x & 63;
    // opaque at each issue, so that the offsets below are formed here and not hoisted
    // out of the loop (and spilled)
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int qb = 0; qb < C::MASK_BLOCKS; ++qb) {
      if (qb < cm.blocks) {
        const int ql = qb * 64 + lane < cm.qn ? qb * 64 + lane : 0;
        const uint32_t voff = (uint32_t)(((cm.q0 + ql) * cm.kv_len + t0) >> 3);
        dma<false>(slot + qb * 512, voff, cm.seg);
        dma<false>(slot + qb * 512 + 256, voff + 4, cm.seg);
      }
    }
  }
}

// This lane's visibility bits of keys t0 + 8j .. t0 + 8j + 7 for the query of its row
// `row` (tile-local), from the step's slot of the mask ring; keys after tlast hidden.
template <int DK, int DV, int FMT>
__device__ __forceinline__ uint32_t coop_mask_bits(const CoopMask& cm, int row, int j, int G,
                                                   int q0, int64_t kv_len, int kv0, int t0,
                                                   int tlast) {
  using C = CoopShape<DK, DV, FMT>;
  const int nvalid = tlast - (t0 + 8 * j) + 1;
  const uint32_t keep = nvalid <= 0 ? 0u : (nvalid >= 8 ? 0xFFu : (1u << nvalid) - 1u);
  const int ql = min(row / G, C::MASK_BLOCKS * 64 - 1);  // rows past the tile are not stored
  const uint32_t at = cm.ring + (((t0 - kv0) >> 5) & 3) * C::MASK_SLOT + (ql >> 6) * 512 +
                      (ql & 63) * 4;
  uint32_t lo, hi;
  lds_load<4>(at, &lo);
  lds_load<4>(at + 256, &hi);
  const int sh = (int)(((int64_t)(q0 + ql) * kv_len + kv0) & 7) + 8 * j;
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  return ((uint32_t)(v >> sh) & 0xFFu) & keep;
}

// Q quarter-row multiplied by the score factor c (the scores then leave the product in
// base-2 exponent units) and rounded to fp16, relative error at most 2^-12 per
// element.  Returns false when the row could overflow fp16 (|q c| >= 2^15, or not
// finite): the caller then takes the exact prescaled form of load_q_operand.
template <int DK>
__device__ __forceinline__ bool load_q_scaled(const uint16_t* qrow, bool valid, int j, float c,
                                              f16x8 (&qf)[DK / 32]) {
  constexpr int QW = DK / 8;
  uint32_t qraw[QW];
  if (valid) {
    load_bytes<DK / 2>(reinterpret_cast<const uint8_t*>(qrow + j * (DK / 4)), qraw);
  } else {
#pragma unroll
    for (int i = 0; i < QW; ++i) qraw[i] = 0u;
  }
  // the largest magnitude as the largest sign-cleared bit pattern (see load_q_operand)
  typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
  u16x2 mb = {0, 0};
#pragma unroll
  for (int i = 0; i < QW; ++i)
    mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, qraw[i] & 0x7FFF7FFFu));
  const float qmax = __uint_as_float((uint32_t)(mb[0] > mb[1] ? mb[0] : mb[1]) << 16);
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    f16x2 p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w = qraw[4 * s + t];
      p[t] = f16x2{(_Float16)(bf16f(w & 0xFFFF) * c), (_Float16)(bf16f(w >> 16) * c)};
    }
    qf[s] = pack8(p[0], p[1], p[2], p[3]);
  }
  return qmax * c < 32768.f;
}

// Softmax with the reference point inside the product (head dims up to 256).  Q carries
// the score factor, and each row group's QK accumulators start at -r, where r is the
// row's reference point (0 while the row has seen no key): the products then give
// x = c s - r directly and p = exp2(x), without a multiply-add per score.  A row moves
// its reference when its largest x passes the slack, and at its first visible key: in
// a step whose keys every row sees (no mask) that can only be the item's first step,
// where every row moves; a masked step also moves rows that have no reference yet.
struct ShiftRef {
  f32x4 negr;
  __device__ __forceinline__ void init() { negr = f32x4{0.f, 0.f, 0.f, 0.f}; }
};

// Under a wave-uniform branch taken when some lane of the group voted (see ShiftRef):
// moves the reference of the rows whose largest score passed the slack, or that had
// none, rescales their accumulators and row sums, and shifts this step's x to the new
// reference.
template <int NT>
__device__ __forceinline__ void raise_shifted(RowState<NT, AccForm::VGPR>& st, ShiftRef& sr,
                                              float bm, float (&x)[8]) {
  const float r = -sr.negr[0];
  const float bmr = max_over_groups(bm) + r;  // the row's largest c s
  const bool up = bmr > st.m + kRescaleSlack;
  const float m_new = up ? bmr : st.m;
  const float alpha = up ? fast_exp2(st.m - m_new) : 1.f;  // 0 when m was -inf
#pragma unroll
  for (int e = 0; e < NT; e += 4)
    scale16(st.acc[e], st.acc[e + 1], st.acc[e + 2], st.acc[e + 3], alpha);
  st.l *= alpha;
  st.m = m_new;
  const float r_new = m_new == -INFINITY ? 0.f : m_new;
  const float d = r_new - r;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] -= d;
  sr.negr = f32x4{-r_new, -r_new, -r_new, -r_new};
}

// P = exp2(x) in fp16 and the lane's row sum of those fp16 values.
template <int NT>
__device__ __forceinline__ f16x8 probs_shifted(RowState<NT, AccForm::VGPR>& st, const float (&x)[8]) {
  f16x2 pp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pp[i] = f16x2{(_Float16)fast_exp2(x[2 * i]), (_Float16)fast_exp2(x[2 * i + 1])};
  const f16x2 one2 = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) st.l = __builtin_amdgcn_fdot2(pp[i], one2, st.l, false);
  return pack8(pp[0], pp[1], pp[2], pp[3]);
}

// CMASK: the launch carries a custom mask (AttnArgs::mask); ROPE: Q and K are rotated
// (AttnArgs::rope); SMALL: pages of 1..8 tokens (per-lane copy addresses from page-table
// entries streamed into LDS slots, see ring_issue_small).  Separate instantiations, so
// that the plain kernel holds none of their state.
template <int DK, int DV, int FMT, bool CMASK, bool ROPE, bool SMALL = false>
__global__ __launch_bounds__((CoopShape<DK, DV, FMT>::NW * 64))
__attribute__((amdgpu_waves_per_eu(CoopShape<DK, DV, FMT>::WGS_PER_CU)))
void prefill_coop_kernel(AttnArgs a) {
  using S = StepShape<DK, DV, FMT>;
  using C = CoopShape<DK, DV, FMT>;
  constexpr int NR = C::NR;
  constexpr int WL = 3 * C::RAW_STAGE;
  static_assert(C::OK, "shape has no cooperative kernel");
  static_assert(!(CMASK && ROPE), "RoPE is not combined with custom masks");
  constexpr int LDS_BASE = CMASK ? C::LDS_MASKED : (ROPE ? C::LDS_ROPE : C::LDS);
  constexpr int LDS = LDS_BASE + (SMALL ? kCoopEntryBytes : 0);
  static_assert(LDS == coop_lds_formula(DK, DV, FMT, CMASK, ROPE, SMALL) &&
                C::WGS_PER_CU == coop_wgs_per_cu(DK, DV), "LDS formula");
  constexpr bool PIECE = C::piece(ROPE);
  static_assert(LDS * C::WGS_PER_CU <= kLdsPerCu, "resident workgroups exceed the LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4;
  const int n = lane & 15;
  const int32_t* rec = a.work + (int64_t)blockIdx.x * kWorkFields;
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.part_scale = a.out_scale;  // for the merge
  const int b = rec[W_REQ], kvh = rec[W_KVH], q0 = rec[W_ROW0], qn = rec[W_ROWS];
  const int kv0 = rec[W_KV0], kv1 = rec[W_KV1], slot = rec[W_SLOT];
  const int G = a.group;
  const int Rn = qn * G;
  const int row_base = wave * NR * 16;
  const int qstart = a.qo_indptr[b];
  const int qlen = a.qo_indptr[b + 1] - qstart;
  const int off = a.kv_lens[b] - qlen;

  f16x8 qf[NR][S::NS];
  float sc[NR];
  bool rv[NR];
  int64_t tokrow[NR];
  int headi[NR];
  const uint16_t* qrows[NR];
  float qpos_f[NR];
  // keys the tile needs: up to the last visible key of its last row
  const int tile_end = a.causal ? min(kv1, q0 + (Rn - 1) / G + off + 1) : kv1;
  const int tlast = kv1 - 1;
  const int nsteps = tile_end > kv0 ? (tile_end - kv0 + kDecodeStep - 1) / kDecodeStep : 0;

  PagedView<DK, DV, true, FMT> view;
  view.init(a, b, kvh, lane);
  CoopCopies<DK, DV, FMT> cc;
  {
    RingPlan<DK, DV, WL, FMT> rp;
    rp.init(lane, view.k_tok, view.v_tok, view.ksf_tok, view.vsf_tok);
    if constexpr (PIECE) cc.rotate_k(rp, lane);
    cc.init(rp, wave);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  const uint32_t raw0 = lds0, opb0 = lds0 + 3 * C::RAW_STAGE;
  // custom mask (the plan tiles the whole key range then: every step is masked)
  constexpr bool custom = CMASK;
  const int64_t kv_len = a.kv_lens[b];
  CoopMask cm;
  cm.seg = nullptr;
  cm.blocks = 0;
  cm.ring = opb0 + 2 * C::OPB;
  cm.q0 = q0;
  cm.kv_len = kv_len;
  cm.qn = qn;
  if constexpr (CMASK) {
    cm.seg = a.mask + a.mask_off[b];
    cm.blocks = (qn + 63) / 64;
  }
  // RoPE: the frequency table after the operand buffers (visible to the dequantisation
  // after the prologue's barrier)
  const uint32_t rope_tab = opb0 + 2 * C::OPB;
  if constexpr (ROPE) {
    if (threadIdx.x < DK)
      *(__attribute__((address_space(3))) float*)(size_t)(rope_tab + 4 * threadIdx.x) =
          a.rope[threadIdx.x];
  }
  CoopLanes<DK, DV, FMT, ROPE> cl;
  cl.init(wave, lane, rope_tab);
  uint32_t bad = 0;

  // SMALL: the page-table entries of a wave's copies, four slots per copy role after the
  // rest of the LDS; the first three steps' entries are read here, at once (the later
  // ones go out with the copies, three steps ahead).
  uint32_t ids = lds0 + LDS_BASE + (uint32_t)(wave & 3) * 1024;
  if constexpr (SMALL) {
    if (wave < 3 && nsteps > 0) {
      for (int m = 0; m < 3; ++m)
        small_entries(ids + (uint32_t)m * 256, view.pt_row, kv0 + m * kDecodeStep, tlast,
                      view.page_shift, lane);
      small_wait<0>(ids);
    }
  }
  // The first three steps' copies go out before Q is read, so that the two memory
  // latencies of a work item's start overlap.
  for (int i = 0; i < 3 && i < nsteps; ++i)
    coop_issue<DK, DV, FMT, CMASK, SMALL, PIECE>(wave, cc, raw0 + i * C::RAW_STAGE, view,
                                                 kv0 + i * kDecodeStep, tlast, bad, cm, kv0, ids);
  // Head dims up to 256: Q carries the score factor (see ShiftRef) unless some row of
  // the wave could overflow fp16; that wave then takes the exact prescaled Q.
  bool safe = true;
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    const int r = row_base + rg * 16 + n;
    rv[rg] = r < Rn;
    const int qi = r / G;
    const int gh = r - qi * G;
    const int qpos = q0 + qi;
    tokrow[rg] = (int64_t)qstart + qpos;
    headi[rg] = kvh * G + gh;
    const uint16_t* qrow = a.q + tokrow[rg] * a.q_s_row + (int64_t)headi[rg] * a.q_s_head;
    if constexpr (ROPE) {
      qrows[rg] = qrow;
      qpos_f[rg] = (float)(qpos + off);  // the query's position
    } else {
      safe = load_q_scaled<DK>(qrow, rv[rg], j, a.score_scale, qf[rg]) && safe;
    }
  }
  // RoPE: all rows rotated together (scaled by the score factor, as load_q_scaled, unless
  // the wide kernel, which takes the exact prescaled form)
  auto rope_prescaled = [&]() {
    float mul[NR], amax[NR];
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      int qexp = 0;
      const float qmax = q_row_absmax<DK>(qrows[rg], rv[rg], j);
      if (qmax > 0.f) (void)frexpf(qmax, &qexp);
      mul[rg] = ldexpf(1.f, 15 - qexp);
      sc[rg] = a.score_scale * ldexpf(1.f, qexp - 15);
    }
    load_q_rope_rows<DK, NR, C::WGS_PER_CU == 1>(qrows, rv, j, qpos_f, a.rope, mul, qf, amax);
  };
  if constexpr (ROPE && C::WIDE) {
    rope_prescaled();
  } else if constexpr (ROPE) {
    float mul[NR], amax[NR];
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) mul[rg] = a.score_scale;
    load_q_rope_rows<DK, NR, C::WGS_PER_CU == 1>(qrows, rv, j, qpos_f, a.rope, mul, qf, amax);
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) safe = amax[rg] < 32768.f && safe;
  }
  // (the rotary wide kernel keeps the exact prescaled Q and the plain softmax)
  constexpr bool SHIFTABLE = !(ROPE && C::WIDE);
  const bool shifted = SHIFTABLE && __all(safe);
  if (SHIFTABLE && !shifted) {
    if constexpr (ROPE) {
      rope_prescaled();
    } else {
#pragma unroll
      for (int rg = 0; rg < NR; ++rg)
        sc[rg] = a.score_scale *
                 load_q_operand<DK>(a.q + tokrow[rg] * a.q_s_row + (int64_t)headi[rg] * a.q_s_head,
                                    rv[rg], j, qf[rg]);
    }
  }

  // One wave per SIMD (wide heads): the Q operands are only ever MFMA sources, so they
  // are kept in AGPRs, leaving the VGPRs to the accumulators and the step's operands.
  // Two waves per SIMD: everything fits the 256 VGPRs of a wave.
  if constexpr (C::WGS_PER_CU == 1) {
#pragma unroll
    for (int rg = 0; rg < NR; ++rg)
#pragma unroll
      for (int s = 0; s < S::NS; ++s) asm volatile("" : "+a"(qf[rg][s]));
  }

  RowState<S::NT, AccForm::VGPR> st[NR];
  ShiftRef sr[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    st[rg].init();
    sr[rg].init();
  }

  auto t_of = [&](int i) { return kv0 + i * kDecodeStep; };
  // the last key row group rg may see; recomputed in the (few) masked steps rather than
  // held in registers for the whole loop
  auto last_of = [&](int rg) {
    const int qpos = q0 + (row_base + rg * 16 + n) / G;
    return a.causal ? min(kv1 - 1, qpos + off) : kv1 - 1;
  };
  // One step: wait for the next raw step, refill the ring, dequantise the next step
  // and compute this one.  MASK: some key of the step is past some row's limit.
  auto step = [&](int i, auto mask_tag, auto shift_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool SHIFT = decltype(shift_tag)::value && SHIFTABLE;
    const bool next = i + 1 < nsteps;
    // raw step i+1 landed (only step i+2 may still be in flight); operands of step i
    // are visible; nobody reads operand buffer (i+1)%2 or raw stage i%3 any more
    if (next) coop_wait<DK, DV, FMT, SMALL>(wave, i + 2 < nsteps, 2 * cm.blocks);
    __syncthreads();
    if (i + 3 < nsteps)
      coop_issue<DK, DV, FMT, CMASK, SMALL, PIECE>(wave, cc, raw0 + (i % 3) * C::RAW_STAGE, view,
                                                   t_of(i + 3), tlast, bad, cm, kv0, ids);
    // Stage and buffer bases as single scalars: left to itself the compiler folds the
    // modulo's parts into every lane address separately (two vector adds per address).
    const uint32_t ob = __builtin_amdgcn_readfirstlane(opb0 + (i & 1) * C::OPB);
    const int t0 = t_of(i);
    const uint32_t obl = ob + lane * 16;  // this lane's entry of operand 0
    const uint32_t rs = __builtin_amdgcn_readfirstlane(raw0 + ((i + 1) % 3) * C::RAW_STAGE);
    const uint32_t ob1 = __builtin_amdgcn_readfirstlane(opb0 + ((i + 1) & 1) * C::OPB);
    if constexpr (C::WIDE) {
      // The two waves of a SIMD take the step's two parts in opposite orders: one
      // dequantises its share of the next step and then computes this one, the other
      // computes first, so that one wave's vector and LDS work runs beside the other's
      // products.  The one barrier a step covers both orders.  Waves w and w + 4 share a
      // SIMD when waves are placed round robin, w and w + 1 when in pairs: this split
      // separates both.
      const bool late = ((wave ^ (wave >> 2)) & 1) != 0;  // uniform
      auto dequant_next = [&]() {
        if (!next) return;
        if (t_of(i + 1) + kDecodeStep - 1 > tlast)
          coop_dequant<DK, DV, true, FMT, ROPE>(rs, ob1, wave, cl, tlast - t_of(i + 1),
                                                (float)t_of(i + 1));
        else
          coop_dequant<DK, DV, false, FMT, ROPE>(rs, ob1, wave, cl, 0, (float)t_of(i + 1));
      };
      if (!late) dequant_next();
      f32x4 sa[NR], sb[NR];
#pragma unroll
      for (int rg = 0; rg < NR; ++rg) {
        sa[rg] = SHIFT ? sr[rg].negr : f32x4{0.f, 0.f, 0.f, 0.f};
        sb[rg] = sa[rg];
      }
      // K operands PF - 1 k-steps ahead of their products, the order pinned by
      // scheduling groups: left to itself the compiler moves every read next to its
      // product (three operand registers instead of PF) and each pair of products
      // then waits for the LDS.
      constexpr int PF = kWidePrefetch;
      f16x8 ka[PF], kb[PF];
      auto kload = [&](int s) {
        lds_load<16>(obl + s * 1024, reinterpret_cast<uint32_t*>(&ka[s % PF]));
        lds_load<16>(obl + (S::NS + s) * 1024, reinterpret_cast<uint32_t*>(&kb[s % PF]));
      };
      __builtin_amdgcn_s_setprio(1);  // the QK products first, as below
#pragma unroll
      for (int s = 0; s < PF - 1; ++s) kload(s);
#pragma unroll
      for (int s = 0; s < S::NS; ++s) {
        if (s + PF - 1 < S::NS) kload(s + PF - 1);
#pragma unroll
        for (int rg = 0; rg < NR; ++rg) {
          sa[rg] = mfma16x16x32(ka[s % PF], qf[rg][s], sa[rg]);
          sb[rg] = mfma16x16x32(kb[s % PF], qf[rg][s], sb[rg]);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PF - 1), 0);
#pragma unroll
      for (int s = 0; s < S::NS; ++s) {
        if (s + PF - 1 < S::NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NR, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      // softmax as in the narrower kernels: scores, the rare reference move, then P
      float x[NR][8], bm[NR];
      const bool first = i == 0;  // uniform
      auto vote = [&](int rg) -> bool {
        if constexpr (SHIFT)
          return first || bm[rg] > kRescaleSlack || (MASK && st[rg].m == -INFINITY);
        else
          return st[rg].wants(bm[rg], sc[rg]);
      };
      uint64_t want = 0;
#pragma unroll
      for (int rg = 0; rg < NR; ++rg) {
        if (MASK && custom)
          bm[rg] = st[rg].scores_vis(sa[rg], sb[rg],
                                     coop_mask_bits<DK, DV, FMT>(cm, row_base + rg * 16 + n, j, G, q0,
                                                                 kv_len, kv0, t0, tlast),
                                     x[rg]);
        else
          bm[rg] = st[rg].template scores<MASK>(sa[rg], sb[rg], t0, j, MASK ? last_of(rg) : 0, x[rg]);
        want |= __ballot(vote(rg));
      }
      if (want != 0) {
#pragma unroll
        for (int rg = 0; rg < NR; ++rg) {
          if (__ballot(vote(rg)) != 0) {
            if constexpr (SHIFT)
              raise_shifted(st[rg], sr[rg], bm[rg], x[rg]);
            else
              st[rg].raise(bm[rg], sc[rg]);
          }
        }
      }
      f16x8 p[NR];
#pragma unroll
      for (int rg = 0; rg < NR; ++rg)
        p[rg] = SHIFT ? probs_shifted(st[rg], x[rg]) : st[rg].template probs<MASK>(x[rg], sc[rg]);
      f16x8 vt[PF];
      auto vload = [&](int e) {
        lds_load<16>(obl + (2 * S::NS + e) * 1024, reinterpret_cast<uint32_t*>(&vt[e % PF]));
      };
#pragma unroll
      for (int e = 0; e < PF - 1; ++e) vload(e);
#pragma unroll
      for (int e = 0; e < S::NT; ++e) {
        if (e + PF - 1 < S::NT) vload(e + PF - 1);
#pragma unroll
        for (int rg = 0; rg < NR; ++rg)
          st[rg].acc[e] = mfma16x16x32(vt[e % PF], p[rg], st[rg].acc[e]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, PF - 1, 0);
#pragma unroll
      for (int e = 0; e < S::NT; ++e) {
        if (e + PF - 1 < S::NT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NR, 0);
      }
      if (late) dequant_next();
      return;
    }
    // Two straight-line blocks.  The first reads this step's K operands and the next
    // step's raw bytes, forms S = K Q^T for every row group and dequantises the next
    // step beside those products (on the last step: a stale stage, into the operand
    // buffer nobody reads any more), then takes each row group's largest score.  The
    // rare rescale sits between the blocks; the second forms P and O^T += V^T P^T for
    // every row group, each group's PV products beside the next group's exponentials.
    f16x8 ka[S::NS], kb[S::NS], vt[S::NT];
    // This block at raised wave priority: of the two workgroups sharing a SIMD, the
    // wave that is issuing its QK products goes first and the other wave's softmax and
    // PV work fills the matrix unit's gaps (about 4 % faster than equal priorities;
    // raising the PV block as well, or the barrier and copy issue, gained nothing).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < S::NS; ++s) {
      lds_load<16>(obl + s * 1024, reinterpret_cast<uint32_t*>(&ka[s]));
      lds_load<16>(obl + (S::NS + s) * 1024, reinterpret_cast<uint32_t*>(&kb[s]));
    }
    CoopRaw<DK, DV, FMT, ROPE> raw;
    raw.load(rs, wave, cl);
    f32x4 sa[NR], sb[NR];
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      sa[rg] = SHIFT ? sr[rg].negr : f32x4{0.f, 0.f, 0.f, 0.f};
      sb[rg] = sa[rg];
#pragma unroll
      for (int s = 0; s < S::NS; ++s) {
        sa[rg] = mfma16x16x32(ka[s], qf[rg][s], sa[rg]);
        sb[rg] = mfma16x16x32(kb[s], qf[rg][s], sb[rg]);
      }
    }
    raw.template store<true>(ob1, wave, cl, tlast - t_of(i + 1), (float)t_of(i + 1));
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int e = 0; e < S::NT; ++e)
      lds_load<16>(obl + (2 * S::NS + e) * 1024, reinterpret_cast<uint32_t*>(&vt[e]));
    float x[NR][8], bm[NR];
    const bool first = i == 0;  // uniform
    auto vote = [&](int rg) -> bool {
      if constexpr (SHIFT)
        return first || bm[rg] > kRescaleSlack || (MASK && st[rg].m == -INFINITY);
      else
        return st[rg].wants(bm[rg], sc[rg]);
    };
    uint64_t want = 0;  // the groups' votes, combined as wave masks on the scalar unit
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      if (MASK && custom)
        bm[rg] = st[rg].scores_vis(sa[rg], sb[rg],
                                   coop_mask_bits<DK, DV, FMT>(cm, row_base + rg * 16 + n, j, G, q0,
                                                               kv_len, kv0, t0, tlast),
                                   x[rg]);
      else
        bm[rg] = st[rg].template scores<MASK>(sa[rg], sb[rg], t0, j, MASK ? last_of(rg) : 0, x[rg]);
      want |= __ballot(vote(rg));
    }
    if (want != 0) {
#pragma unroll
      for (int rg = 0; rg < NR; ++rg) {
        if (__ballot(vote(rg)) != 0) {
          if constexpr (SHIFT)
            raise_shifted(st[rg], sr[rg], bm[rg], x[rg]);
          else
            st[rg].raise(bm[rg], sc[rg]);
        }
      }
    }
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      const f16x8 p = SHIFT ? probs_shifted(st[rg], x[rg]) : st[rg].template probs<MASK>(x[rg], sc[rg]);
      st[rg].pv(vt, p);
    }
    // order of the second block: group 0's P, then one PV product of group g to a share
    // of group g+1's P (16 VALU instructions a group shifted, 24 otherwise), then the
    // last group's products
    constexpr int PV_VALU = SHIFT ? 2 : 3;
    __builtin_amdgcn_sched_group_barrier(0x002, SHIFT ? 16 : 20, 0);
#pragma unroll
    for (int rg = 1; rg < NR; ++rg)
#pragma unroll
      for (int e = 0; e < S::NT; ++e) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, PV_VALU, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x008, S::NT, 0);
  };
  // prologue: three steps in flight (issued above), step 0 dequantised
  if (nsteps > 0) {
    coop_wait<DK, DV, FMT, SMALL>(wave, false, 2 * cm.blocks);
    __syncthreads();
    coop_dequant<DK, DV, true, FMT, ROPE>(raw0, opb0, wave, cl, tlast - t_of(0), (float)t_of(0));
  }
  // steps whose 32 keys are visible to every row of the tile, then the rest
  const int tile_min_last = a.causal ? min(kv1 - 1, q0 + off) : kv1 - 1;
  const int n_full = custom ? 0 : min(nsteps, max(0, (tile_min_last - kv0 + 1) / kDecodeStep));
  int i = 0;
  if (shifted) {
    for (; i < n_full; ++i) step(i, std::false_type{}, std::true_type{});
    for (; i < nsteps; ++i) step(i, std::true_type{}, std::true_type{});
  } else {
    for (; i < n_full; ++i) step(i, std::false_type{}, std::false_type{});
    for (; i < nsteps; ++i) step(i, std::true_type{}, std::false_type{});
  }

  const bool badw = __any(bad != 0);
  // the four waves saw different copies: any bad page poisons the whole tile
  __shared__ uint32_t bad_flag;
  if (threadIdx.x == 0) bad_flag = 0;
  __syncthreads();
  if (badw && lane == 0) atomicOr(&bad_flag, 1u);
  __syncthreads();
  const bool bad_any = bad_flag != 0;
  if (row_base >= Rn) return;
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) {
    if (slot < 0) {
      st[rg].store(a.o + tokrow[rg] * a.o_s_row + (int64_t)headi[rg] * a.o_s_head,
                   a.lse + tokrow[rg] * a.num_qo_heads + headi[rg], rv[rg], bad_any, a.out_scale, j);
    } else {
      const int r = row_base + rg * 16 + n;
      st[rg].store_partial(a.part_o + ((int64_t)slot * a.rows_per_slot + r) * DV,
                   a.part_lse + (int64_t)slot * a.rows_per_slot + r, rv[rg], bad_any, j);
    }
  }
}

// ROPE: the rotary kernels (a.rope set; never with a custom mask); else the plain or
// custom-mask ones.
template <int DK, int DV, int FMT, bool ROPE>
hipError_t launch_dk_dv(int page_shift, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_work);
  const dim3 block(CoopShape<DK, DV, FMT>::NW * 64);
  // pages of 16 tokens or more, or fewer (SMALL)
  if constexpr (ROPE) {
    if (page_shift >= 4)
      launch_attention(prefill_coop_kernel<DK, DV, FMT, false, true>, grid, block, stream, a);
    else
      launch_attention(prefill_coop_kernel<DK, DV, FMT, false, true, true>, grid, block, stream, a);
  } else {
    if (page_shift >= 4 && a.mask)
      launch_attention(prefill_coop_kernel<DK, DV, FMT, true, false>, grid, block, stream, a);
    else if (page_shift >= 4)
      launch_attention(prefill_coop_kernel<DK, DV, FMT, false, false>, grid, block, stream, a);
    else if (a.mask)
      launch_attention(prefill_coop_kernel<DK, DV, FMT, true, false, true>, grid, block, stream, a);
    else
      launch_attention(prefill_coop_kernel<DK, DV, FMT, false, false, true>, grid, block, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

// Shapes with kernels: NVFP4 at every (qk, vo) pair of 64..512 with vo <= qk except
// 512/512; FP8 at head dims up to 256 (the 512/256 FP8 tile needs more LDS than a CU
// has, and the narrower 512-dim FP8 shapes are not built).
#define NVFP4_PREFILL_SHAPES(X)                                                     \
  X(64, 64, kNvfp4) X(128, 64, kNvfp4) X(128, 128, kNvfp4) X(256, 64, kNvfp4)      \
  X(256, 128, kNvfp4) X(256, 256, kNvfp4) X(512, 64, kNvfp4) X(512, 128, kNvfp4)   \
  X(512, 256, kNvfp4) X(64, 64, kFp8) X(128, 64, kFp8) X(128, 128, kFp8)           \
  X(256, 64, kFp8) X(256, 128, kFp8) X(256, 256, kFp8)

}  // namespace nvfp4
