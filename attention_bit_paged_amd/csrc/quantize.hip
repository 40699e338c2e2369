// Quantisation of bf16 K/V rows into a paged pool: NVFP4 (the per-block arithmetic
// and its exactness argument are in fp4_quant.h) or FP8 e4m3 with a per-tensor scale.
#include <algorithm>

#include "fp4_quant.h"
#include "internal.h"

namespace nvfp4 {

namespace {

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
    const int64_t page = slot >> a.page_shift;
    const int64_t off = slot & (((int64_t)1 << a.page_shift) - 1);
    uint8_t* row = a.data + page * a.d_page + head * a.d_head + off * a.d_tok;
    if (a.fp8) {
      // FP8: every element on its own, sign | RNE_e4m3(|x| / g) saturated (exact: see
      // fp4_quant.h, the quotient of a bf16 value by a float cannot land on a midpoint
      // it is not exactly on)
      uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFF;
        const double ax = (double)fabsf(quant::bf16_to_float(bits));
        const uint32_t code = quant::e4m3_code(ax / a.gscale) | ((bits >> 8) & 0x80);
        c[e >> 2] |= code << (8 * (e & 3));
      }
      *reinterpret_cast<uint4*>(row + blk * 16) = make_uint4(c[0], c[1], c[2], c[3]);
      continue;
    }
    uint32_t p0, p1, sc;
    quant::block16(w, a.gscale, p0, p1, sc);
    *reinterpret_cast<uint2*>(row + blk * 8) = make_uint2(p0, p1);
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
