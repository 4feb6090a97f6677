// The transposed operand layouts (DeepGEMM实战 §3.3) with per-row A factors
// (the template article's per-channel factors, §3.4) on the 256-row tiles of
// gemm_fp8_big.h, 256 and 128 columns wide. Its own translation unit, so these
// instances compile beside the others.

#include <hip/hip_runtime.h>

#include "gemm_fp8_big.h"
#include "gemm_fp8_nt.h"

namespace dg {

hipError_t launch_big_layout_rowa(int id, const GemmArgs& p, hipStream_t stream) {
  switch (id) {
    case 4: return big::launch_layout<128, 256, 2, 2>(p, stream);
    case 5: return big::launch_layout<64, 256, 2, 2>(p, stream);
    case 9: return big::launch_layout<128, 128, 4, 2>(p, stream);
    case 10: return big::launch_layout<64, 128, 4, 2>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
