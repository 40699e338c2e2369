// NVFP4 quantisation of bf16 K/V rows into a paged pool.
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
#include <algorithm>

#include "internal.h"

namespace nvfp4 {

namespace {

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

// One thread per 16-element block.  IDX: the index type, 32-bit whenever the block
// count allows (64-bit division is a long software sequence on the GPU).
template <typename IDX>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs ka, QuantArgs va,
                                                       int64_t n_tokens,
                                                       const int64_t* __restrict__ slots) {
  const QuantArgs& a = blockIdx.y == 0 ? ka : va;
  const int blocks_per_row = a.head_dim / 16;
  const IDX total = (IDX)(n_tokens * a.num_heads * blocks_per_row);
  for (IDX idx = (IDX)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (IDX)gridDim.x * blockDim.x) {
    const int blk = (int)(idx % blocks_per_row);
    const IDX th = idx / blocks_per_row;
    const int head = (int)(th % a.num_heads);
    const int64_t tok = (int64_t)(th / a.num_heads);
    // the source row and the slot are loaded together (one memory round trip)
    const uint4* src = reinterpret_cast<const uint4*>(a.src + tok * a.s_tok + head * a.s_head +
                                                      blk * 16);
    const int64_t slot = slots[tok];
    const uint4 u0 = src[0];
    const uint4 u1 = src[1];
    if (slot < 0 || slot >= a.num_slots) continue;
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      amax = fmaxf(amax, fabsf(bf16_to_float(w[i] & 0xFFFF)));
      amax = fmaxf(amax, fabsf(bf16_to_float(w[i] >> 16)));
    }
    const uint32_t sc = e4m3_code((double)amax / (6.0 * a.gscale));
    const double sg = e4m3_value(sc) * a.gscale;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFF);
      const double ax = (double)fabsf(bf16_to_float(bits));
      uint32_t nib = sc == 0 ? 0u : e2m1_code(ax, sg);
      nib |= (bits >> 12) & 0x8;              // sign bit of x
      packed[i >> 3] |= nib << (4 * (i & 7));
    }
    const int64_t page = slot >> a.page_shift;
    const int64_t off = slot & (((int64_t)1 << a.page_shift) - 1);
    uint2* dst = reinterpret_cast<uint2*>(a.data + page * a.d_page + head * a.d_head +
                                          off * a.d_tok + blk * 8);
    *dst = make_uint2(packed[0], packed[1]);
    a.sf[page * a.sf_page + head * a.sf_head + off * a.sf_tok + blk] = (uint8_t)sc;
  }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs* k, const QuantArgs* v, int64_t n_tokens,
                           const int64_t* slots, hipStream_t stream) {
  const QuantArgs& first = k ? *k : *v;
  const QuantArgs& second = (k && v) ? *v : first;
  const int ny = (k && v) ? 2 : 1;
  const int64_t per = n_tokens * (int64_t)std::max(first.num_heads * first.head_dim,
                                                   second.num_heads * second.head_dim) / 16;
  int64_t nb = (per + 255) / 256;
  if (nb > 65535 * 8) nb = 65535 * 8;
  if (nb < 1) nb = 1;
  if (per + (int64_t)nb * 256 < ((int64_t)1 << 31))
    hipLaunchKernelGGL(quantize_kernel<int32_t>, dim3((unsigned)nb, ny), dim3(256), 0, stream,
                       first, second, n_tokens, slots);
  else
    hipLaunchKernelGGL(quantize_kernel<int64_t>, dim3((unsigned)nb, ny), dim3(256), 0, stream,
                       first, second, n_tokens, slots);
  return hipGetLastError();
}

}  // namespace nvfp4
