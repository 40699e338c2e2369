// In-kernel RoPE of the prefill kernels: rotation of Q rows at load and of K operand
// pairs in the cooperative dequantisation.
#pragma once

#include "attn_step.h"

namespace nvfp4 {

// ------------------------------------------------------------------ RoPE --
// Rotate-half rotary embedding ([PF] commit "Address CodeRabbit review on
// flashinfer-ai#3684 (5 findings)", item init_rope_freq: one frequency per pair of QK
// head-dim elements, half the QK dim of them).  Element i < D/2 of a Q or K row and
// element i + D/2 turn together by the angle pos * w_i.  A frequency comes as a float
// pair (hi, lo) with hi + lo = w_i / (2 pi), in turns per position.

// cos and sin of the angle pos * (hi + lo) turns.  The whole turns drop out before
// any rounding that matters: the fma recovers the rounding error of pos * hi exactly,
// so the fraction of a turn keeps about 24 bits at any position below 2^24 (a plain
// float product would lose one bit of it per doubling of the position).  The
// hardware sin / cos take their argument in turns.
__device__ __forceinline__ void rope_cs(float pos, float hi, float lo, float& c, float& s) {
  const float p = pos * hi;
  const float t = __builtin_amdgcn_fractf(p) + fmaf(pos, lo, fmaf(pos, hi, -p));
  c = __builtin_amdgcn_cosf(t);
  s = __builtin_amdgcn_sinf(t);
}

// Largest |q| of a query row (over the four lane groups of its column).
template <int DK>
__device__ __forceinline__ float q_row_absmax(const uint16_t* qrow, bool valid, int j) {
  constexpr int QW = DK / 8;
  uint32_t qraw[QW];
  if (valid) {
    load_bytes<DK / 2>(reinterpret_cast<const uint8_t*>(qrow + j * (DK / 4)), qraw);
  } else {
#pragma unroll
    for (int i = 0; i < QW; ++i) qraw[i] = 0u;
  }
  float qmax = 0.f;
#pragma unroll
  for (int i = 0; i < QW; ++i)
    qmax = fmaxf(qmax, fmaxf(fabsf(bf16f(qraw[i] & 0xFFFF)), fabsf(bf16f(qraw[i] >> 16))));
  return max_over_groups(qmax);
}

// The Q quarter-rows of a wave's NR row groups rotated, k-step by k-step: a k-step's
// eight frequency pairs are read once for all rows, and a row's own and partner loads
// are issued one k-step at a time (all of them at once held every row's quarter-rows
// beside the kernel's state and spilled it).  Row rg is scaled by mul[rg]; amax[rg]
// returns its largest |rotated q * mul| (NaN when an input is NaN).  AGPR: each operand
// moves to the accumulation registers as soon as it is made (kernels that keep Q there).
template <int DK, int NR, bool AGPR = false>
__device__ __forceinline__ void load_q_rope_rows(const uint16_t* const (&qrow)[NR],
                                                 const bool (&valid)[NR], int j,
                                                 const float (&pos)[NR], const float* freq,
                                                 const float (&mul)[NR], f16x8 (&qf)[NR][DK / 32],
                                                 float (&amax)[NR]) {
  const float* fr = freq + 2 * ((j & 1) * (DK / 4));
  const float sgn = j < 2 ? -1.f : 1.f;  // first half: x cos - y sin; second: x cos + y sin
#pragma unroll
  for (int rg = 0; rg < NR; ++rg) amax[rg] = 0.f;
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    uint32_t fw[16];
    load_bytes<64>(reinterpret_cast<const uint8_t*>(fr + 16 * s), fw);
#pragma unroll
    for (int rg = 0; rg < NR; ++rg) {
      uint32_t xo[4] = {0u, 0u, 0u, 0u}, xp[4] = {0u, 0u, 0u, 0u};
      if (valid[rg]) {
        load_bytes<16>(reinterpret_cast<const uint8_t*>(qrow[rg] + j * (DK / 4)) + 16 * s, xo);
        load_bytes<16>(reinterpret_cast<const uint8_t*>(qrow[rg] + (j ^ 2) * (DK / 4)) + 16 * s,
                       xp);
      }
      f16x2 p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float r[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float x = bf16f(h ? xo[t] >> 16 : xo[t] & 0xFFFF);
          const float y = bf16f(h ? xp[t] >> 16 : xp[t] & 0xFFFF);
          float c, sn;
          rope_cs(pos[rg], __builtin_bit_cast(float, fw[2 * (2 * t + h)]),
                  __builtin_bit_cast(float, fw[2 * (2 * t + h) + 1]), c, sn);
          r[h] = fmaf(x, c, sgn * (y * sn)) * mul[rg];
          amax[rg] = __builtin_elementwise_maximum(amax[rg], fabsf(r[h]));
        }
        p[t] = f16x2{(_Float16)r[0], (_Float16)r[1]};
      }
      qf[rg][s] = pack8(p[0], p[1], p[2], p[3]);
      if constexpr (AGPR) asm volatile("" : "+a"(qf[rg][s]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Rotates one pair of K operand vectors in place: lo holds elements i .. i+7 of a key
// row (pair indices i0 .. i0+7), hi the partner elements i + D/2 ...; `tab` the LDS
// address of the pairs' eight frequencies.
__device__ __forceinline__ void rope_k_pair(f16x8& lo, f16x8& hi, float pos, uint32_t tab) {
  // plain float loads (merged into 16-byte reads): element reads of a loaded vector
  // that is then bit cast can take element 0 whatever the index
  typedef __attribute__((address_space(3))) const float* lds_f32;
  float fw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) fw[i] = ((lds_f32)(size_t)tab)[i];
  f16x2 a[4], b[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float ra[2], rb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * t + h;
      const float x1 = (float)lo[e], x2 = (float)hi[e];
      float c, sn;
      rope_cs(pos, fw[2 * e], fw[2 * e + 1], c, sn);
      ra[h] = fmaf(x1, c, -(x2 * sn));
      rb[h] = fmaf(x2, c, x1 * sn);
    }
    a[t] = f16x2{(_Float16)ra[0], (_Float16)ra[1]};
    b[t] = f16x2{(_Float16)rb[0], (_Float16)rb[1]};
  }
  lo = pack8(a[0], a[1], a[2], a[3]);
  hi = pack8(b[0], b[1], b[2], b[3]);
}

}  // namespace nvfp4
