// Per-wave LDS ring for streaming paged NVFP4 K/V (page_size >= 16).
//
// Each stage holds the raw bytes of one 32-token step: K rows, V rows, K scales and V
// scales, each token-major.  The bytes are copied by gfx950's direct global-to-LDS
// loads (64 lanes x 16 or 4 bytes per instruction, placed in lane order at the LDS
// address held in m0), so several steps are in flight without spending registers.
// The copies are issued through inline assembly and waited for with explicit vmcnt
// counts: inside the streaming loop they are the wave's only vector-memory
// operations, so "the newest n steps may still be in flight" is an exact count.
// [XQA] "Support NVFP4 KV cache decode on SM120", changelog: packed K/V and their
// scale factors are staged on chip before the unpack (there through shared memory
// with grain-sized copies; here through this ring).
#pragma once

#include "attn_step.h"

namespace nvfp4 {

template <int DK, int DV>
struct RingShape {
  static constexpr int KD = 16 * DK;  // 32 tokens x DK/2 bytes
  static constexpr int VD = 16 * DV;
  static constexpr int KS = 2 * DK;   // 32 tokens x DK/16 scale bytes
  static constexpr int VS = 2 * DV;
  static constexpr int OFF_KD = 0;
  static constexpr int OFF_VD = KD;
  static constexpr int OFF_SF = KD + VD;  // K scales, then V scales
  static constexpr int SFP = (KS + VS + 255) / 256 * 256;  // scale region, padded
  static constexpr int STAGE = KD + VD + SFP;
  static constexpr int N_KD = KD / 1024;  // 16-byte-per-lane copies
  static constexpr int N_VD = VD / 1024;
  static constexpr int N_SF = SFP / 256;  // 4-byte-per-lane copies
  static constexpr int NDMA = N_KD + N_VD + N_SF;
  // stages per wave: as many as fit 76 KiB per workgroup of four waves, 2..4
  static constexpr int NST_RAW = (76 * 1024) / (4 * STAGE);
  static constexpr int NST = NST_RAW < 2 ? 2 : (NST_RAW > 4 ? 4 : NST_RAW);
  static constexpr int WAVE_BYTES = NST * STAGE;
  static_assert(KD % 1024 == 0 && VD % 1024 == 0, "ring shape");
  static_assert(NDMA * (NST - 1) <= 63, "vmcnt range");
};

// The copies are not declared to touch memory: they only write this wave's ring, which
// is read after an explicit wait whose result (a zero) feeds the read addresses, so the
// compiler cannot hoist those reads above it.  Keeping the global view unclobbered lets
// the page-table reads stay scalar loads.
__device__ __forceinline__ void dma16(uint32_t lds_addr, const uint8_t* src) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_addr), "v"(src));
}
__device__ __forceinline__ void dma4(uint32_t lds_addr, const uint8_t* src) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_addr), "v"(src));
}
template <int N>
__device__ __forceinline__ uint32_t wait_vm() {
  uint32_t zero;
  asm volatile("s_waitcnt vmcnt(%1)\n\ts_mov_b32 %0, 0" : "=s"(zero) : "n"(N));
  return zero;
}
// Wait until at most `newer` steps of NDMA copies each are still in flight.  Returns 0.
template <int NDMA, int NST>
__device__ __forceinline__ uint32_t wait_steps(int newer) {
  if (NST > 3 && newer >= 3) return wait_vm<NDMA * 3 <= 63 ? NDMA * 3 : 63>();
  if (NST > 2 && newer >= 2) return wait_vm<NDMA * 2 <= 63 ? NDMA * 2 : 63>();
  if (newer >= 1) return wait_vm<NDMA <= 63 ? NDMA : 63>();
  return wait_vm<0>();
}

// Per-lane copy plan of one stage: for every copy instruction, which pool, which
// 16-token half and which byte offset inside that half this lane fetches.
template <int DK, int DV>
struct RingPlan {
  using R = RingShape<DK, DV>;
  uint32_t off[R::NDMA];     // byte offset from the half's base
  uint32_t sel[R::NDMA];     // bit 0: second half; bit 1: V pool (scale copies only)

  // token strides in bytes: k_tok/v_tok (data), ks_tok/vs_tok (scales)
  __device__ __forceinline__ void init(int lane, int64_t k_tok, int64_t v_tok, int64_t ks_tok,
                                       int64_t vs_tok) {
#pragma unroll
    for (int i = 0; i < R::N_KD; ++i) {
      const int byte = i * 1024 + lane * 16;
      const int t = byte / (DK / 2), in_row = byte % (DK / 2);
      off[i] = (uint32_t)((t & 15) * k_tok) + in_row;
      sel[i] = t >= 16;
    }
#pragma unroll
    for (int i = 0; i < R::N_VD; ++i) {
      const int byte = i * 1024 + lane * 16;
      const int t = byte / (DV / 2), in_row = byte % (DV / 2);
      off[R::N_KD + i] = (uint32_t)((t & 15) * v_tok) + in_row;
      sel[R::N_KD + i] = t >= 16;
    }
#pragma unroll
    for (int i = 0; i < R::N_SF; ++i) {
      int byte = i * 256 + lane * 4;
      if (byte >= R::KS + R::VS) {  // padding: re-read a valid dword, land past the scales
        off[R::N_KD + R::N_VD + i] = 0;
        sel[R::N_KD + R::N_VD + i] = 0;
        continue;
      }
      const bool vpool = byte >= R::KS;
      if (vpool) byte -= R::KS;
      const int row = vpool ? DV / 16 : DK / 16;
      const int t = byte / row, in_row = byte % row;
      off[R::N_KD + R::N_VD + i] = (uint32_t)((t & 15) * (vpool ? vs_tok : ks_tok)) + in_row;
      sel[R::N_KD + R::N_VD + i] = (t >= 16 ? 1u : 0u) | (vpool ? 2u : 0u);
    }
  }
};

// Issues the copies of the step starting at token t0 into the stage at lds_stage.
// Bases of the two 16-token halves come from two page-table entries; a half that
// starts after tlast reuses the first half's page (its bytes are never used).
template <int DK, int DV>
__device__ __forceinline__ void ring_issue(const RingPlan<DK, DV>& rp, uint32_t lds_stage,
                                           const PagedView<DK, DV, true>& pv, int t0, int tlast,
                                           uint32_t& bad) {
  using R = RingShape<DK, DV>;
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
  const uint8_t* kb[2] = {at(pv.kdat, pg0, s0, pv.k_page, pv.k_tok), at(pv.kdat, pg1, s1, pv.k_page, pv.k_tok)};
  const uint8_t* vb[2] = {at(pv.vdat, pg0, s0, pv.v_page, pv.v_tok), at(pv.vdat, pg1, s1, pv.v_page, pv.v_tok)};
  const uint8_t* ksb[2] = {at(pv.ksf, pg0, s0, pv.ksf_page, pv.ksf_tok),
                           at(pv.ksf, pg1, s1, pv.ksf_page, pv.ksf_tok)};
  const uint8_t* vsb[2] = {at(pv.vsf, pg0, s0, pv.vsf_page, pv.vsf_tok),
                           at(pv.vsf, pg1, s1, pv.vsf_page, pv.vsf_tok)};
  // the previous reads of this stage were consumed already; make sure they completed
  asm volatile("s_waitcnt lgkmcnt(0)");
#pragma unroll
  for (int i = 0; i < R::N_KD; ++i)
    dma16(lds_stage + R::OFF_KD + i * 1024, (rp.sel[i] ? kb[1] : kb[0]) + rp.off[i]);
#pragma unroll
  for (int i = 0; i < R::N_VD; ++i) {
    const int c = R::N_KD + i;
    dma16(lds_stage + R::OFF_VD + i * 1024, (rp.sel[c] ? vb[1] : vb[0]) + rp.off[c]);
  }
#pragma unroll
  for (int i = 0; i < R::N_SF; ++i) {
    const int c = R::N_KD + R::N_VD + i;
    const uint32_t s = rp.sel[c];
    const uint8_t* base = (s & 2) ? ((s & 1) ? vsb[1] : vsb[0]) : ((s & 1) ? ksb[1] : ksb[0]);
    dma4(lds_stage + R::OFF_SF + i * 256, base + rp.off[c]);
  }
}

// Reads a step's raw bytes for this lane from an LDS stage, in the register layout the
// step helpers expect (the same as a direct load from the pool).
template <int DK, int DV>
__device__ __forceinline__ void ring_read(const uint8_t* stage, int j, int n, StepRaw<DK, DV>& r) {
  using R = RingShape<DK, DV>;
  using S = StepShape<DK, DV>;
  const int ta = 8 * (n >> 2) + (n & 3);
  const int tb = ta + 4;
  load_bytes<S::KB>(stage + R::OFF_KD + ta * (DK / 2) + j * S::KB, r.ka);
  load_bytes<S::KB>(stage + R::OFF_KD + tb * (DK / 2) + j * S::KB, r.kb);
  load_bytes<S::KSF>(stage + R::OFF_SF + ta * (DK / 16) + j * S::KSF, r.ksa);
  load_bytes<S::KSF>(stage + R::OFF_SF + tb * (DK / 16) + j * S::KSF, r.ksb);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = 8 * j + i;
    load_bytes<S::VB>(stage + R::OFF_VD + t * (DV / 2) + n * S::VB, r.vd[i]);
    load_bytes<S::VSFB>(stage + R::OFF_SF + R::KS + t * (DV / 16) + (n * DV / 16) / 16, &r.vs[i]);
  }
}

}  // namespace nvfp4
