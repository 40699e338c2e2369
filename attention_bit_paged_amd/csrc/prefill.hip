// Host side of the paged prefill: the shapes with kernels, their LDS and tile sizes,
// and the launch (RoPE launches are built in prefill_rope.hip).
#include <algorithm>

#include "prefill_kernels.h"

namespace nvfp4 {
bool prefill_supported(int dk, int dv, int fmt) {
#define NVFP4_PREFILL_CASE(K, V, F) \
  if (dk == K && dv == V && fmt == F) return true;
  NVFP4_PREFILL_SHAPES(NVFP4_PREFILL_CASE)
#undef NVFP4_PREFILL_CASE
  return false;
}

int prefill_wgs_per_cu(int dk, int dv) { return dk <= 128 && dv <= 128 ? 2 : 1; }

int prefill_rows_per_item(int dk, int dv, int /*group*/, int /*page_size*/) {
  if ((dk <= 256 && dv <= 256) || (dk == 512 && dv <= 256))
    return dk <= 128 && dv <= 128 ? 192 : 128;  // cooperative kernel: 4 waves x NR x 16 rows
  return 64 * (dk >= 512 ? 1 : 2);
}

size_t prefill_lds_bytes(int dk, int dv, int page_size, int fmt) {
  // the resident workgroups of the cooperative kernel (its larger form: custom-mask or
  // RoPE; pages below 16 tokens add the entry slots), also for shapes without one
  const bool small = page_size < 16;
  const int most = std::max(coop_lds_formula(dk, dv, fmt, true, false, small),
                            coop_lds_formula(dk, dv, fmt, false, true, small));
  return (size_t)most * coop_wgs_per_cu(dk, dv);
}

hipError_t launch_prefill(int dk, int dv, int fmt, int page_shift, const AttnArgs& a,
                          hipStream_t stream) {
  if (a.n_work <= 0) return hipSuccess;
  if (a.rope) return launch_prefill_rope(dk, dv, fmt, page_shift, a, stream);
#define NVFP4_PREFILL_CASE(K, V, F) \
  if (dk == K && dv == V && fmt == F) return launch_dk_dv<K, V, F, false>(page_shift, a, stream);
  NVFP4_PREFILL_SHAPES(NVFP4_PREFILL_CASE)
#undef NVFP4_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
