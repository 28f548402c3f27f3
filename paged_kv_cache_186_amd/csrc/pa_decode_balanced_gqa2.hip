// Balanced-split paged decode for grouped-query attention (gfx950), every
// K/V tile load serving 2 query heads (fp16 / bf16 queries, 16-bit or 8-bit
// caches).  The kernel template and its description are in
// pa_balanced_kernel.h.

#include "pa_balanced_kernel.h"

namespace pa {

hipError_t launch_decode_balanced_gqa2(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == PA_DTYPE_F16 ? run_balanced_kv<F16, 2>(a, stream)
                                 : run_balanced_kv<BF16, 2>(a, stream);
}

}  // namespace pa
