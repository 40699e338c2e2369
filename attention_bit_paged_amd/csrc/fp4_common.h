// Device helpers shared by the attention kernels: NVFP4 -> fp16 dequantisation,
// MFMA wrappers and wave reductions for gfx950.
//
// Dequantisation: every e2m1 x e4m3 product has at most 2 + 4 significant bits
// and lies in [2^-10, 2688], so it is exact in fp16.  The hardware fp4 -> f16
// converter applies only the exponent of its scale operand, so it is called with
// scale 1.0 and the e4m3 block scale (converted exactly to fp16) is applied with a
// packed fp16 multiply.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two e2m1 values (byte BYTE of w: low nibble first) -> exact fp16 pair.
template <int BYTE>
__device__ __forceinline__ f16x2 fp4x2_to_f16(uint32_t w) {
  return __builtin_bit_cast(f16x2, __builtin_bit_cast(uint32_t,
      __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, BYTE)));
}

// Two e4m3fn bytes (bytes 0,1 when HI is false, else 2,3) -> exact fp16 pair.
template <bool HI>
__device__ __forceinline__ f16x2 fp8x2_to_f16(uint32_t w) {
  return __builtin_bit_cast(f16x2, __builtin_bit_cast(uint32_t,
      __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI)));
}

__device__ __forceinline__ uint32_t f16x2_bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ f16x8 pack8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  u32x4 u = {f16x2_bits(a), f16x2_bits(b), f16x2_bits(c), f16x2_bits(d)};
  return __builtin_bit_cast(f16x8, u);
}

// Eight consecutive e2m1 elements of one row (one dword) times one scale.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 scale) {
  return pack8(fp4x2_to_f16<0>(w) * scale, fp4x2_to_f16<1>(w) * scale,
               fp4x2_to_f16<2>(w) * scale, fp4x2_to_f16<3>(w) * scale);
}

__device__ __forceinline__ f16x2 splat_lo(f16x2 v) { return f16x2{v[0], v[0]}; }
__device__ __forceinline__ f16x2 splat_hi(f16x2 v) { return f16x2{v[1], v[1]}; }

// D[16x16] += A[16x32] * B[32x16]; lane l holds A row l%16 / B column l%16,
// k-slots 8*(l/16)..+7, and D rows 4*(l/16)..+3 of column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four k-groups of one column).
// gfx950's permlane swaps exchange 16-lane rows (odd rows of the first operand with
// even rows of the second) and 32-lane halves; with both operands holding v, the two
// results hold {v[l], v[l^16]} (resp. {v[l], v[l^32]}) in some order on every lane.
// The results are copied out as plain integers before the bit casts: a bit cast of a
// vector element directly reads element 0 whatever the index.
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
// v_max_f32 as is: fmaxf on values the compiler cannot prove canonical adds a
// quieting v_max of each input first.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_over_groups(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(max_raw(a, b), a, b);
  return max_raw(a, b);
}
__device__ __forceinline__ float sum_over_groups(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(a + b, a, b);
  return a + b;
}

// Unaligned-size loads of N bytes (N in {1, 2, 4, 8, 16}) into dwords.
template <int N>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t* out) {
  if constexpr (N == 1) {
    out[0] = *p;
  } else if constexpr (N == 2) {
    out[0] = *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (N == 4) {
    out[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (N == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = v.x;
    out[1] = v.y;
  } else {
    static_assert(N % 16 == 0, "load size");
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      out[4 * i + 0] = v.x;
      out[4 * i + 1] = v.y;
      out[4 * i + 2] = v.z;
      out[4 * i + 3] = v.w;
    }
  }
}

// bf16 bits -> float.
__device__ __forceinline__ float bf16f(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

}  // namespace nvfp4
