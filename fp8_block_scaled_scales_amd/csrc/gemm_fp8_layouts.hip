// The transposed operand layouts of the block-scaled FP8 GEMM (DeepGEMM实战
// §3.3: A and B may each be stored transposed, [K,M] and [K,N], and are read
// that way without a transposed copy in memory): the tiled and split-K
// kernels of gemm_fp8_tiled.h with a transposed tile staged as K rows and
// read with the transposing LDS read. Its own translation unit, so these
// instances compile beside the NT ones.

#include <hip/hip_runtime.h>

#include "gemm_fp8_nt.h"
#include "gemm_fp8_tiled.h"

namespace dg {

// g x g A factors here; per-row A factors in gemm_fp8_layouts_rowa.hip.
hipError_t launch_layout(int id, const GemmArgs& p, hipStream_t stream) {
  if (p.rowa) return launch_layout_rowa(id, p, stream);
  switch (id) {
    case 0: return launch_tiled_layout<128, 128, 2, 2, 2, 128, 4, false, 1>(p, stream);
    case 1: return launch_tiled_layout<128, 128, 2, 2, 2, 64, 4, false, 1>(p, stream);
    case 2: return launch_tiled_layout<64, 64, 2, 2, 8, 128, 4, true, 1>(p, stream);
    case 3: return launch_tiled_layout<64, 64, 2, 2, 8, 64, 4, true, 1>(p, stream);
    default: return launch_big_layout(id, p, stream);
  }
}

}  // namespace dg
