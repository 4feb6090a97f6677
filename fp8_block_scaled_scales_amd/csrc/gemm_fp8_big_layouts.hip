// The transposed operand layouts (DeepGEMM实战 §3.3: A stored [K,M], B
// stored [K,N], read that way without a transposed copy) on the 256-row tiles
// of gemm_fp8_big.h, 256 and 128 columns wide. Its own translation unit, so
// these instances compile beside the NT ones.

#include <hip/hip_runtime.h>

#include "gemm_fp8_big.h"
#include "gemm_fp8_nt.h"

namespace dg {

// g x g A factors here; per-row A factors in gemm_fp8_big_layouts_rowa.hip.
hipError_t launch_big_layout(int id, const GemmArgs& p, hipStream_t stream) {
  switch (id) {
    case 4: return big::launch_layout<128, 256, 2, 1>(p, stream);
    case 5: return big::launch_layout<64, 256, 2, 1>(p, stream);
    case 9: return big::launch_layout<128, 128, 4, 1>(p, stream);
    case 10: return big::launch_layout<64, 128, 4, 1>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
