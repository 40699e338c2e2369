// Per-wave LDS ring for streaming paged NVFP4 K/V (page_size >= 16).
//
// Each stage holds the raw bytes of one 32-token step: K rows, V rows, K scales and V
// scales, each token-major.  The bytes are copied by gfx950's direct global-to-LDS
// loads (64 lanes x 16 or 4 bytes per instruction, placed in lane order at the LDS
// address held in m0), so several steps are in flight without spending registers.
// Every copy takes its 64-bit base from SGPRs and a loop-invariant 32-bit offset per
// lane, so issuing a step costs no vector instructions: a copy whose lanes fall into
// several (pool, 16-token half) groups is issued once per group under an exec mask.
// The copies are waited for with explicit vmcnt counts: inside the streaming loop they
// are the wave's only vector-memory operations, so "the newest n steps may still be in
// flight" is an exact count.
// [XQA] "Support NVFP4 KV cache decode on SM120", changelog: packed K/V and their
// scale factors are staged on chip before the unpack (there through shared memory
// with grain-sized copies; here through this ring).
#pragma once

#include <utility>

#include "attn_step.h"

namespace nvfp4 {

// WAVE_LDS: LDS bytes available to one wave's ring; the ring is 2..4 stages deep.
// FMT: the pools' storage format (FP8 rows are twice as long and have no scale rows).
template <int DK, int DV, int FMT = kNvfp4>
struct RingBytes {
  using S = StepShape<DK, DV, FMT>;
  static constexpr int KD = 32 * S::RBK;  // 32 tokens of K rows
  static constexpr int VD = 32 * S::RBV;
  static constexpr int KS = 32 * S::SBK;  // 32 tokens of K scale rows (0 for FP8)
  static constexpr int VS = 32 * S::SBV;
  static constexpr int SFP = (KS + VS + 255) / 256 * 256;  // scale region, padded
  static constexpr int STAGE = KD + VD + SFP;
};

template <int DK, int DV, int WAVE_LDS, int FMT = kNvfp4>
struct RingShape {
  using S = StepShape<DK, DV, FMT>;
  static constexpr int RBK = S::RBK, RBV = S::RBV;
  // scale row bytes (FP8 has none: every scale branch below is then unreachable, and the
  // divisor is kept nonzero)
  static constexpr int SBK = S::SBK > 0 ? S::SBK : 1, SBV = S::SBV > 0 ? S::SBV : 1;
  static constexpr int KD = 32 * RBK;
  static constexpr int VD = 32 * RBV;
  static constexpr int KS = 32 * S::SBK;
  static constexpr int VS = 32 * S::SBV;
  static constexpr int OFF_KD = 0;
  static constexpr int OFF_VD = KD;
  static constexpr int OFF_SF = KD + VD;  // K scales, then V scales
  static constexpr int SFP = (KS + VS + 255) / 256 * 256;  // scale region, padded
  static constexpr int STAGE = KD + VD + SFP;
  static constexpr int N_KD = KD / 1024;  // 16-byte-per-lane copies
  static constexpr int N_VD = VD / 1024;
  static constexpr int N_SF = SFP / 256;  // 4-byte-per-lane copies
  static constexpr int NCOPY = N_KD + N_VD + N_SF;
  static_assert(KD % 1024 == 0 && VD % 1024 == 0, "ring shape");

  // Group of the bytes lane `lane` moves in copy c: 0/1 K rows of token half 0/1,
  // 2/3 V rows, 4/5 K scales, 6/7 V scales; -1 for padding lanes (not issued).
  static constexpr int group(int c, int lane) {
    if (c < N_KD) return (c * 1024 + lane * 16) / RBK >= 16 ? 1 : 0;
    if (c < N_KD + N_VD) return ((c - N_KD) * 1024 + lane * 16) / RBV >= 16 ? 3 : 2;
    int byte = (c - N_KD - N_VD) * 256 + lane * 4;
    if (byte >= KS + VS) return -1;
    if (byte < KS) return byte / SBK >= 16 ? 5 : 4;
    byte -= KS;
    return byte / SBV >= 16 ? 7 : 6;
  }
  static constexpr uint64_t mask(int c, int g) {
    uint64_t m = 0;
    for (int l = 0; l < 64; ++l)
      if (group(c, l) == g) m |= uint64_t(1) << l;
    return m;
  }
  // copy instructions per stage for the pools in the bit set `pools` (bit 0 K rows,
  // 1 V rows, 2 K scales, 3 V scales)
  static constexpr int ndma(int pools = 0xF) {
    int n = 0;
    for (int c = 0; c < NCOPY; ++c)
      for (int g = 0; g < 8; ++g) n += ((pools >> (g / 2)) & 1) && mask(c, g) != 0;
    return n;
  }
  static constexpr int lds_off(int c) {
    return c < N_KD ? OFF_KD + c * 1024
                    : (c < N_KD + N_VD ? OFF_VD + (c - N_KD) * 1024
                                       : OFF_SF + (c - N_KD - N_VD) * 256);
  }
  static constexpr int NDMA = ndma(0xF);  // copy instructions per stage
  static constexpr int NST_RAW = WAVE_LDS / STAGE;
  static constexpr int NST = NST_RAW > 4 ? 4 : NST_RAW;
  static_assert(NST >= 2, "LDS budget below two stages");
  static constexpr int WAVE_BYTES = NST * STAGE;
  static_assert(NDMA * (NST - 1) <= 63, "vmcnt range");
};

// m0 must be written one instruction ahead of the copy that reads it.  The copies are
// not declared to touch memory: they only write this wave's ring, whose reads take
// their addresses from the wait below, so the compiler cannot move them above it.
// Keeping the global view unclobbered lets the page-table reads stay scalar loads.
// NT: the copy carries the non-temporal cache policy, for bytes that one launch reads
// once (decode): they then do not displace from the caches what is read again, the
// work records, the page table and the partial rows.
// A flag beside the pool bits of ring_issue: the step's copies take the non-temporal
// policy.
constexpr int kStreamCopies = 0x10;
#define NVFP4_DMA_X4(nt) "s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" nt
#define NVFP4_DMA_X1(nt) "s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" nt
template <bool X4, bool NT = false>
__device__ __forceinline__ void dma(uint32_t m0, uint32_t voff, const uint8_t* sbase) {
  if constexpr (X4 && NT)
    asm volatile(NVFP4_DMA_X4(" nt") :: "s"(m0), "v"(voff), "s"(sbase));
  else if constexpr (X4)
    asm volatile(NVFP4_DMA_X4("") :: "s"(m0), "v"(voff), "s"(sbase));
  else if constexpr (NT)
    asm volatile(NVFP4_DMA_X1(" nt") :: "s"(m0), "v"(voff), "s"(sbase));
  else
    asm volatile(NVFP4_DMA_X1("") :: "s"(m0), "v"(voff), "s"(sbase));
}
// The same copy for the lanes in (LO, HI) only; exec is restored inside the statement.
#define NVFP4_DMA_MASKED(op, nt)                                                        \
  "s_mov_b64 %0, exec\n\ts_mov_b32 exec_lo, %4\n\ts_mov_b32 exec_hi, %5\n\t"            \
  "s_mov_b32 m0, %1\n\ts_nop 0\n\t" op " %2, %3" nt "\n\ts_mov_b64 exec, %0"
template <bool X4, int LO, int HI, bool NT = false>
__device__ __forceinline__ void dma_masked(uint32_t m0, uint32_t voff, const uint8_t* sbase) {
  uint64_t save;
  if constexpr (X4 && NT)
    asm volatile(NVFP4_DMA_MASKED("global_load_lds_dwordx4", " nt")
                 : "=&s"(save) : "s"(m0), "v"(voff), "s"(sbase), "n"(LO), "n"(HI));
  else if constexpr (X4)
    asm volatile(NVFP4_DMA_MASKED("global_load_lds_dwordx4", "")
                 : "=&s"(save) : "s"(m0), "v"(voff), "s"(sbase), "n"(LO), "n"(HI));
  else if constexpr (NT)
    asm volatile(NVFP4_DMA_MASKED("global_load_lds_dword", " nt")
                 : "=&s"(save) : "s"(m0), "v"(voff), "s"(sbase), "n"(LO), "n"(HI));
  else
    asm volatile(NVFP4_DMA_MASKED("global_load_lds_dword", "")
                 : "=&s"(save) : "s"(m0), "v"(voff), "s"(sbase), "n"(LO), "n"(HI));
}
#undef NVFP4_DMA_X4
#undef NVFP4_DMA_X1
#undef NVFP4_DMA_MASKED

// LDS byte addresses of this lane's reads in stage 0 of its wave's ring.  They pass
// through every wait (tied asm operands), which both orders the reads after the wait
// and lets each read use one base register plus an immediate offset.
struct RingLanes {
  uint32_t k, ks, v, vs;
};

template <int N>
__device__ __forceinline__ void ring_wait(RingLanes& b) {
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(b.k), "+v"(b.ks), "+v"(b.v), "+v"(b.vs) : "n"(N));
}
// Waits for vmcnt(N) when `newer` is set (wave-uniform), else for vmcnt(0).
template <int N>
__device__ __forceinline__ void ring_wait_sel(RingLanes& b, uint32_t newer) {
  asm volatile("s_cmp_eq_u32 %4, 0\n\ts_cbranch_scc1 1f\n\ts_waitcnt vmcnt(%5)\n\ts_branch 2f\n"
               "1:\n\ts_waitcnt vmcnt(0)\n2:"
               : "+v"(b.k), "+v"(b.ks), "+v"(b.v), "+v"(b.vs)
               : "s"(__builtin_amdgcn_readfirstlane(newer)), "n"(N)
               : "scc");
}

// Per-lane copy offsets of one stage, relative to the lane's group base.
template <int DK, int DV, int WAVE_LDS, int FMT = kNvfp4>
struct RingPlan {
  using R = RingShape<DK, DV, WAVE_LDS, FMT>;
  uint32_t off[R::NCOPY];

  // token strides in bytes: k_tok/v_tok (data), ks_tok/vs_tok (scales); the host
  // keeps 16 token strides plus a row inside 32 bits
  __device__ __forceinline__ void init(int lane, int64_t k_tok, int64_t v_tok, int64_t ks_tok,
                                       int64_t vs_tok) {
#pragma unroll
    for (int i = 0; i < R::N_KD; ++i) {
      const int byte = i * 1024 + lane * 16;
      const int t = byte / R::RBK, in_row = byte % R::RBK;
      off[i] = (uint32_t)(t & 15) * (uint32_t)k_tok + in_row;
    }
#pragma unroll
    for (int i = 0; i < R::N_VD; ++i) {
      const int byte = i * 1024 + lane * 16;
      const int t = byte / R::RBV, in_row = byte % R::RBV;
      off[R::N_KD + i] = (uint32_t)(t & 15) * (uint32_t)v_tok + in_row;
    }
#pragma unroll
    for (int i = 0; i < R::N_SF; ++i) {
      int byte = i * 256 + lane * 4;
      uint32_t o = 0;
      if (byte < R::KS) {
        o = (uint32_t)((byte / R::SBK) & 15) * (uint32_t)ks_tok + byte % R::SBK;
      } else if (byte < R::KS + R::VS) {
        byte -= R::KS;
        o = (uint32_t)((byte / R::SBV) & 15) * (uint32_t)vs_tok + byte % R::SBV;
      }
      off[R::N_KD + R::N_VD + i] = o;
    }
  }
};

namespace ring_detail {

template <int DK, int DV, int WL, int FMT, int POOLS, int C, int G>
__device__ __forceinline__ void issue_group(uint32_t m0, uint32_t voff,
                                            const uint8_t* const (&base)[8]) {
  using R = RingShape<DK, DV, WL, FMT>;
  constexpr uint64_t M = ((POOLS >> (G / 2)) & 1) ? R::mask(C, G) : 0;
  constexpr bool X4 = C < R::N_KD + R::N_VD;
  constexpr bool NT = (POOLS & kStreamCopies) != 0;
  if constexpr (M == ~uint64_t(0)) {
    dma<X4, NT>(m0, voff, base[G]);
  } else if constexpr (M != 0) {
    dma_masked<X4, (int)(uint32_t)M, (int)(uint32_t)(M >> 32), NT>(m0, voff, base[G]);
  }
}

template <int DK, int DV, int WL, int FMT, int POOLS, int C>
__device__ __forceinline__ void issue_copy(uint32_t stage_lds, const RingPlan<DK, DV, WL, FMT>& rp,
                                           const uint8_t* const (&base)[8]) {
  using R = RingShape<DK, DV, WL, FMT>;
  const uint32_t m0 = stage_lds + R::lds_off(C);
  issue_group<DK, DV, WL, FMT, POOLS, C, 0>(m0, rp.off[C], base);
  issue_group<DK, DV, WL, FMT, POOLS, C, 1>(m0, rp.off[C], base);
  issue_group<DK, DV, WL, FMT, POOLS, C, 2>(m0, rp.off[C], base);
  issue_group<DK, DV, WL, FMT, POOLS, C, 3>(m0, rp.off[C], base);
  issue_group<DK, DV, WL, FMT, POOLS, C, 4>(m0, rp.off[C], base);
  issue_group<DK, DV, WL, FMT, POOLS, C, 5>(m0, rp.off[C], base);
  issue_group<DK, DV, WL, FMT, POOLS, C, 6>(m0, rp.off[C], base);
  issue_group<DK, DV, WL, FMT, POOLS, C, 7>(m0, rp.off[C], base);
}

template <int DK, int DV, int WL, int FMT, int POOLS, int... Cs>
__device__ __forceinline__ void issue_all(std::integer_sequence<int, Cs...>, uint32_t stage_lds,
                                          const RingPlan<DK, DV, WL, FMT>& rp,
                                          const uint8_t* const (&base)[8]) {
  (issue_copy<DK, DV, WL, FMT, POOLS, Cs>(stage_lds, rp, base), ...);
}

}  // namespace ring_detail

// Issues the copies of the step starting at token t0 into the stage at lds_stage, for
// the pools in the bit set POOLS (see RingShape::ndma), with the non-temporal policy
// when POOLS holds kStreamCopies and the view allows it (a uniform branch).  Bases of
// the two 16-token halves come from two page-table entries; a half that starts after
// tlast reuses the first half's page (its bytes are never used).
template <int DK, int DV, int WL, int POOLS = 0xF, int FMT = kNvfp4>
__device__ __forceinline__ void ring_issue(const RingPlan<DK, DV, WL, FMT>& rp, uint32_t lds_stage,
                                           const PagedView<DK, DV, true, FMT>& pv, int t0,
                                           int tlast, uint32_t& bad) {
  using R = RingShape<DK, DV, WL, FMT>;
  // The page table is read-only while the kernel runs: reading it through the
  // constant address space keeps these uniform reads scalar loads.
  const __attribute__((address_space(4))) int32_t* pt =
      (const __attribute__((address_space(4))) int32_t*)pv.pt_row;
  auto page = [&](int idx) {
    int pg = pt[idx];
    if ((unsigned)pg >= (unsigned)pv.num_pages) {
      bad = 1;
      pg = 0;
    }
    return pg;
  };
  const int pg0 = page(t0 >> pv.page_shift);
  const int s0 = t0 & pv.page_mask;
  const bool h1 = t0 + 16 <= tlast;
  const int pg1 = h1 ? page((t0 + 16) >> pv.page_shift) : pg0;
  const int s1 = h1 ? ((t0 + 16) & pv.page_mask) : s0;
  // strides are below 2^31 (checked by the host): 32 x 32 -> 64-bit products
  auto at = [](const uint8_t* base, int pg, int sl, int64_t page_stride, int64_t tok_stride) {
    return base + (int64_t)pg * (int32_t)page_stride + (int64_t)sl * (int32_t)tok_stride;
  };
  const uint8_t* const base[8] = {
      at(pv.kdat, pg0, s0, pv.k_page, pv.k_tok),     at(pv.kdat, pg1, s1, pv.k_page, pv.k_tok),
      at(pv.vdat, pg0, s0, pv.v_page, pv.v_tok),     at(pv.vdat, pg1, s1, pv.v_page, pv.v_tok),
      at(pv.ksf, pg0, s0, pv.ksf_page, pv.ksf_tok),  at(pv.ksf, pg1, s1, pv.ksf_page, pv.ksf_tok),
      at(pv.vsf, pg0, s0, pv.vsf_page, pv.vsf_tok),  at(pv.vsf, pg1, s1, pv.vsf_page, pv.vsf_tok)};
  // the previous reads of this stage were consumed already; make sure they completed
  asm volatile("s_waitcnt lgkmcnt(0)");
  constexpr int PLAIN = POOLS & ~kStreamCopies;
  if constexpr (PLAIN != POOLS) {
    if (pv.stream) {
      ring_detail::issue_all<DK, DV, WL, FMT, POOLS>(std::make_integer_sequence<int, R::NCOPY>{},
                                                      lds_stage, rp, base);
      return;
    }
  }
  ring_detail::issue_all<DK, DV, WL, FMT, PLAIN>(std::make_integer_sequence<int, R::NCOPY>{},
                                                  lds_stage, rp, base);
}

// LDS addresses of this lane's reads in stage 0 of the ring at ring_lds.
template <int DK, int DV, int WL, int FMT = kNvfp4>
__device__ __forceinline__ RingLanes ring_lanes(uint32_t ring_lds, int j, int n) {
  using R = RingShape<DK, DV, WL, FMT>;
  using S = StepShape<DK, DV, FMT>;
  const int ta = 8 * (n >> 2) + (n & 3);
  RingLanes b;
  b.k = ring_lds + R::OFF_KD + ta * S::RBK + j * S::KB;
  b.ks = ring_lds + R::OFF_SF + ta * S::SBK + j * S::KSF;
  b.v = ring_lds + R::OFF_VD + 8 * j * S::RBV + n * S::VB;
  b.vs = ring_lds + R::OFF_SF + R::KS + 8 * j * S::SBV + (n * DV / 16) / 16;
  return b;
}

template <int N>
__device__ __forceinline__ void lds_load(uint32_t addr, uint32_t* out) {
  typedef __attribute__((address_space(3))) const uint8_t* lds_u8;
  typedef __attribute__((address_space(3))) const uint16_t* lds_u16;
  typedef __attribute__((address_space(3))) const uint32_t* lds_u32;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) const u32x2* lds_u64;
  typedef __attribute__((address_space(3))) const u32x4* lds_u128;
  if constexpr (N == 1) {
    out[0] = *(lds_u8)(size_t)addr;
  } else if constexpr (N == 2) {
    out[0] = *(lds_u16)(size_t)addr;
  } else if constexpr (N == 4) {
    out[0] = *(lds_u32)(size_t)addr;
  } else if constexpr (N == 8) {
    const u32x2 v = *(lds_u64)(size_t)addr;
    out[0] = v[0];
    out[1] = v[1];
  } else {
    static_assert(N % 16 == 0, "load size");
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const u32x4 v = *(lds_u128)(size_t)(addr + 16 * i);
      out[4 * i + 0] = v[0];
      out[4 * i + 1] = v[1];
      out[4 * i + 2] = v[2];
      out[4 * i + 3] = v[3];
    }
  }
}

// ---- pages smaller than a step's 16-token halves (page_size 1..8) ----
//
// A step's 32 tokens then lie on up to 32 pages, so every copy lane forms its own
// 64-bit address from its token's page.  The step's page-table entries reach LDS by a
// copy of their own (one 4-byte entry per lane into a 256-byte slot, some steps before
// the step's data copies need them), so the loop holds no page numbers in registers
// and every vector-memory operation of the stream is still a counted copy.  Each step
// then issues its data copies, one per ring copy and without exec masks (lanes past the
// scale rows fetch token 0's scales into the stage's padding), and one entry copy.
// The copies keep the default cache policy: the prefill kernel that streams them reads
// each request's rows for every query tile.

// Per lane and ring copy C (a constant): the copy's token within the step (t), whether
// it carries a V row or V scale row (isv; scale copies hold both pools' lanes) and the
// byte within the token's row.
template <int DK, int DV, int WL, int FMT, int C>
struct SmallCopy {
  using R = RingShape<DK, DV, WL, FMT>;
  static constexpr bool KD = C < R::N_KD, VD = !KD && C < R::N_KD + R::N_VD;
  int t, in_row;
  bool isv;
  __device__ __forceinline__ explicit SmallCopy(int lane) {
    if constexpr (KD) {
      const int b = C * 1024 + 16 * lane;
      t = b / R::RBK; in_row = b % R::RBK; isv = false;
    } else if constexpr (VD) {
      const int b = (C - R::N_KD) * 1024 + 16 * lane;
      t = b / R::RBV; in_row = b % R::RBV; isv = true;
    } else {
      const int b = (C - R::N_KD - R::N_VD) * 256 + 4 * lane;
      isv = b >= R::KS;
      const int bv = b - R::KS;
      // padding lanes (past both scale regions): token 0's K scales, bytes never read
      const bool pad = bv >= R::VS;
      t = pad ? 0 : (isv ? bv / R::SBV : b / R::SBK);
      in_row = pad ? 0 : (isv ? bv % R::SBV : b % R::SBK);
      isv = isv && !pad;
    }
  }
};

// Loop-invariant part of each copy lane's address: (t mod page_size) * token stride +
// byte in the row (a step starts on a page boundary: its first token is a multiple of
// 16).  Strides are below 2^31 and a page holds at most 8 tokens, so it fits 32 bits
// as the host keeps 16 token strides plus a row there.
template <int DK, int DV, int WL, int FMT = kNvfp4>
struct SmallPlan {
  using R = RingShape<DK, DV, WL, FMT>;
  uint32_t off[R::NCOPY];
  template <int C>
  __device__ __forceinline__ void init_one(int lane, const PagedView<DK, DV, true, FMT>& pv) {
    const SmallCopy<DK, DV, WL, FMT, C> x(lane);
    uint32_t ts;
    if constexpr (SmallCopy<DK, DV, WL, FMT, C>::KD) ts = (uint32_t)pv.k_tok;
    else if constexpr (SmallCopy<DK, DV, WL, FMT, C>::VD) ts = (uint32_t)pv.v_tok;
    else ts = x.isv ? (uint32_t)pv.vsf_tok : (uint32_t)pv.ksf_tok;
    off[C] = (uint32_t)(x.t & pv.page_mask) * ts + (uint32_t)x.in_row;
  }
  template <int... Cs>
  __device__ __forceinline__ void init_all(std::integer_sequence<int, Cs...>, int lane,
                                           const PagedView<DK, DV, true, FMT>& pv) {
    (init_one<Cs>(lane, pv), ...);
  }
  __device__ __forceinline__ void init(int lane, const PagedView<DK, DV, true, FMT>& pv) {
    init_all(std::make_integer_sequence<int, R::NCOPY>{}, lane, pv);
  }
};

// The entry copy of the step at t0 into the slot at LDS `slot`: lane l carries entry
// (t0 >> page_shift) + l, clamped to the entry of key tlast (tlast >= t0).
__device__ __forceinline__ void small_entries(uint32_t slot, const int32_t* pt_row, int t0,
                                              int tlast, int page_shift, int lane) {
  const int e = min((t0 >> page_shift) + lane, tlast >> page_shift);
  dma<false>(slot, (uint32_t)(4 * e), reinterpret_cast<const uint8_t*>(pt_row));
}

// Waits until at most N of the wave's vector-memory operations are in flight; `ids`
// (the entry slot read next) passes through the wait, so the reads follow it.
template <int N>
__device__ __forceinline__ void small_wait(uint32_t& ids) {
  asm volatile("s_waitcnt vmcnt(%1)" : "+s"(ids) : "n"(N));
}

namespace ring_detail {
template <int DK, int DV, int WL, int FMT, int POOLS, int C>
__device__ __forceinline__ void issue_small_copy(const SmallPlan<DK, DV, WL, FMT>& sp,
                                                 uint32_t stage, uint32_t ids,
                                                 const PagedView<DK, DV, true, FMT>& pv,
                                                 int lane, uint32_t& bad) {
  using R = RingShape<DK, DV, WL, FMT>;
  constexpr int MINE = C < R::N_KD ? 1 : (C < R::N_KD + R::N_VD ? 2 : 0xC);
  if constexpr ((POOLS & MINE) == 0) return;
  using X = SmallCopy<DK, DV, WL, FMT, C>;
  const X x(lane);
  uint32_t pg;
  lds_load<4>(ids + 4 * (uint32_t)(x.t >> pv.page_shift), &pg);
  if (pg >= (uint32_t)pv.num_pages) {
    bad = 1;
    pg = 0;
  }
  uint64_t base;
  uint32_t ps;
  if constexpr (X::KD) {
    base = (uint64_t)(uintptr_t)pv.kdat; ps = (uint32_t)pv.k_page;
  } else if constexpr (X::VD) {
    base = (uint64_t)(uintptr_t)pv.vdat; ps = (uint32_t)pv.v_page;
  } else {
    // two-way selects on the lane's pool (a wider select became a table in memory)
    base = x.isv ? (uint64_t)(uintptr_t)pv.vsf : (uint64_t)(uintptr_t)pv.ksf;
    ps = x.isv ? (uint32_t)pv.vsf_page : (uint32_t)pv.ksf_page;
  }
  const uint64_t at = base + (uint64_t)pg * ps + sp.off[C];
  const uint32_t m0 = stage + R::lds_off(C);
  if constexpr (C < R::N_KD + R::N_VD)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(m0), "v"(at));
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(m0), "v"(at));
}
template <int DK, int DV, int WL, int FMT, int POOLS, int... Cs>
__device__ __forceinline__ void issue_small_all(std::integer_sequence<int, Cs...>,
                                                const SmallPlan<DK, DV, WL, FMT>& sp,
                                                uint32_t stage, uint32_t ids,
                                                const PagedView<DK, DV, true, FMT>& pv,
                                                int lane, uint32_t& bad) {
  (issue_small_copy<DK, DV, WL, FMT, POOLS, Cs>(sp, stage, ids, pv, lane, bad), ...);
}
}  // namespace ring_detail

// The data copies of one step into `stage` from the entries in the slot at `ids`, for
// the pools in POOLS (bit 0 K rows, 1 V rows; either scale bit: every scale copy, whose
// lanes carry both pools' rows).  An entry outside [0, num_pages) sets `bad` and reads
// page 0.
template <int DK, int DV, int WL, int POOLS = 0xF, int FMT = kNvfp4>
__device__ __forceinline__ void ring_issue_small(const SmallPlan<DK, DV, WL, FMT>& sp,
                                                 uint32_t stage, uint32_t ids,
                                                 const PagedView<DK, DV, true, FMT>& pv,
                                                 int lane, uint32_t& bad) {
  using R = RingShape<DK, DV, WL, FMT>;
  ring_detail::issue_small_all<DK, DV, WL, FMT, POOLS>(std::make_integer_sequence<int, R::NCOPY>{},
                                                      sp, stage, ids, pv, lane, bad);
}

// Reads a step's raw bytes for this lane from the stage `stage_off` bytes past the
// lane addresses, in the register layout the step helpers expect (the same as a
// direct load from the pool).
template <int DK, int DV, int FMT = kNvfp4>
__device__ __forceinline__ void ring_read(const RingLanes& b, uint32_t stage_off,
                                          StepRaw<DK, DV, FMT>& r) {
  using S = StepShape<DK, DV, FMT>;
  lds_load<S::KB>(b.k + stage_off, r.ka);
  lds_load<S::KB>(b.k + stage_off + 4 * S::RBK, r.kb);
  if constexpr (!S::F8) {
    lds_load<S::KSF>(b.ks + stage_off, r.ksa);
    lds_load<S::KSF>(b.ks + stage_off + 4 * S::SBK, r.ksb);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lds_load<S::VB>(b.v + stage_off + i * S::RBV, r.vd[i]);
    if constexpr (!S::F8) lds_load<S::VSFB>(b.vs + stage_off + i * S::SBV, &r.vs[i]);
  }
}

}  // namespace nvfp4
