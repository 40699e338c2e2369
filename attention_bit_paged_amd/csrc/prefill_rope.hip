// The prefill kernels with in-kernel RoPE, in a translation unit of their own so that
// the two halves of the prefill instantiations compile side by side.
#include "prefill_kernels.h"

namespace nvfp4 {

hipError_t launch_prefill_rope(int dk, int dv, int fmt, int page_shift, const AttnArgs& a,
                               hipStream_t stream) {
#define NVFP4_PREFILL_CASE(K, V, F) \
  if (dk == K && dv == V && fmt == F) return launch_dk_dv<K, V, F, true>(page_shift, a, stream);
  NVFP4_PREFILL_SHAPES(NVFP4_PREFILL_CASE)
#undef NVFP4_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
