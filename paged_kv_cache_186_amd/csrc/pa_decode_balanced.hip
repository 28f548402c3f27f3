// Balanced-split paged decode, one query head per K/V head (gfx950).  The
// kernel template and its description are in pa_balanced_kernel.h.

#include "pa_balanced_kernel.h"

namespace pa {

hipError_t launch_decode_balanced(const DecodeArgs& a, hipStream_t stream) {
  switch (a.group_width) {
    case 2:
      return launch_decode_balanced_gqa2(a, stream);
    case 4:
      return launch_decode_balanced_gqa4(a, stream);
    default:
      break;
  }
  switch (a.dtype) {
    case PA_DTYPE_F32:
      return run_balanced_d<F32, F32, 1>(a, stream);
    case PA_DTYPE_F16:
      return run_balanced_kv<F16, 1>(a, stream);
    default:
      return run_balanced_kv<BF16, 1>(a, stream);
  }
}

}  // namespace pa
