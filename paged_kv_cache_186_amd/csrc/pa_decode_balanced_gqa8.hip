// Balanced-split paged decode for grouped-query attention (gfx950), every
// K/V tile load serving 8 query heads (fp16 / bf16 queries, 16-bit caches
// only: with an 8-bit cache, 8 heads' state does not fit the registers and
// groups of 8 run as two groups of 4).  The kernel template and its
// description are in pa_balanced_kernel.h.

#include "pa_balanced_kernel.h"

namespace pa {

hipError_t launch_decode_balanced_gqa8(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == PA_DTYPE_F16 ? run_balanced_d<F16, F16, 8>(a, stream)
                                 : run_balanced_d<BF16, BF16, 8>(a, stream);
}

}  // namespace pa
