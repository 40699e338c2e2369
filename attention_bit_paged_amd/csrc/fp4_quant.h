// NVFP4 quantisation of one 16-element bf16 block, shared by the append kernel and the
// decode kernel's in-place append of the step's new token.
//
// Format from [PF] "Re-enable split-KV for NVFP4 KV cache in prefill path",
// commit "Gate split-KV off when kv_data_type is NVFP4" (packed uint8, one FP8
// block scale per 16 elements) and [XQA] "Support NVFP4 KV cache decode on SM120",
// changelog (the tests' to_nvfp4 with a global scale).  The scale is amax/6 in e4m3,
// the element the nearest e2m1 value of x/scale.
//
// Decisions are taken in float64, where they are exact: amax is a bf16 value
// (8 significant bits), 6*g is exact, so amax/(6g) rounded to 53 bits can never
// land on the other side of an e4m3 rounding midpoint; each element threshold
// t*s*g has at most 3+4+24 significant bits and is exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {
namespace quant {

// Round-to-nearest-even to e4m3fn for 0 <= q (finite), saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code(double q) {
  if (q >= 448.0) return 0x7E;
  if (q < 0.015625) {                       // below 2^-6: subnormal grid of 2^-9
    return (uint32_t)__builtin_rint(q * 512.0);   // 8 here is the smallest normal, code 0x08
  }
  int e;
  const double f = __builtin_frexp(q, &e);  // q = f * 2^e, f in [0.5, 1)
  const uint32_t m = (uint32_t)__builtin_rint((2.0 * f - 1.0) * 8.0);  // 0..8, 8 carries
  const uint32_t code = ((uint32_t)(e + 6) << 3) + m;
  return code > 0x7E ? 0x7E : code;
}

__device__ __forceinline__ double e4m3_value(uint32_t code) {
  const int ex = (int)(code >> 3) & 0xF;
  const int man = (int)(code & 7);
  if (ex == 0) return __builtin_ldexp((double)man, -9);
  return __builtin_ldexp((double)(8 + man), ex - 10);
}

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Magnitude code of |x| on the e2m1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} scaled by sg.
// A value exactly on a midpoint goes to the even code: the comparison is ">=" at
// midpoints whose upper neighbour has an even code and ">" elsewhere.
__device__ __forceinline__ uint32_t e2m1_code(double a, double sg) {
  uint32_t c = 0;
  c += a > 0.25 * sg;
  c += a >= 0.75 * sg;
  c += a > 1.25 * sg;
  c += a >= 1.75 * sg;
  c += a > 2.5 * sg;
  c += a >= 3.5 * sg;
  c += a > 5.0 * sg;
  return c;
}

// Scale code of a block from its largest magnitude.
__device__ __forceinline__ uint32_t scale_code(float amax, double gscale) {
  return e4m3_code((double)amax / (6.0 * gscale));
}

// Largest magnitude of four bf16 values (two dwords, element 2i in the low half of w[i]).
__device__ __forceinline__ float amax4(uint32_t w0, uint32_t w1) {
  return fmaxf(fmaxf(fabsf(bf16_to_float(w0 & 0xFFFF)), fabsf(bf16_to_float(w0 >> 16))),
               fmaxf(fabsf(bf16_to_float(w1 & 0xFFFF)), fabsf(bf16_to_float(w1 >> 16))));
}

// Codes of four consecutive elements of a block with scale code sc: 16 bits, the first
// element in the low nibble.
__device__ __forceinline__ uint32_t codes4(uint32_t w0, uint32_t w1, uint32_t sc, double gscale) {
  const double sg = e4m3_value(sc) * gscale;
  const uint32_t bits[4] = {w0 & 0xFFFF, w0 >> 16, w1 & 0xFFFF, w1 >> 16};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double ax = (double)fabsf(bf16_to_float(bits[i]));
    uint32_t nib = sc == 0 ? 0u : e2m1_code(ax, sg);
    nib |= (bits[i] >> 12) & 0x8;  // sign bit of x
    out |= nib << (4 * i);
  }
  return out;
}

// The block's 16 bf16 values as eight dwords (element 2i in the low half of w[i]) ->
// eight packed bytes (two dwords, element 0 in the low nibble) and the scale code.
__device__ __forceinline__ void block16(const uint32_t (&w)[8], double gscale, uint32_t& p0,
                                        uint32_t& p1, uint32_t& sc) {
  const float amax = fmaxf(fmaxf(amax4(w[0], w[1]), amax4(w[2], w[3])),
                           fmaxf(amax4(w[4], w[5]), amax4(w[6], w[7])));
  sc = scale_code(amax, gscale);
  p0 = codes4(w[0], w[1], sc, gscale) | (codes4(w[2], w[3], sc, gscale) << 16);
  p1 = codes4(w[4], w[5], sc, gscale) | (codes4(w[6], w[7], sc, gscale) << 16);
}

}  // namespace quant
}  // namespace nvfp4
