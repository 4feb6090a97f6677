// The transposed operand layouts (DeepGEMM实战 §3.3) with per-row A factors
// (one per row of A and K segment, the template article's per-channel factors,
// §3.4) on the tiled and split-K kernels of gemm_fp8_tiled.h. The factors are
// staged per step beside the slabs whatever the storage of A's codes. Its own
// translation unit, so these instances compile beside the others.

#include <hip/hip_runtime.h>

#include "gemm_fp8_nt.h"
#include "gemm_fp8_tiled.h"

namespace dg {

hipError_t launch_layout_rowa(int id, const GemmArgs& p, hipStream_t stream) {
  switch (id) {
    case 0: return launch_tiled_layout<128, 128, 2, 2, 2, 128, 4, false, 2>(p, stream);
    case 1: return launch_tiled_layout<128, 128, 2, 2, 2, 64, 4, false, 2>(p, stream);
    case 2: return launch_tiled_layout<64, 64, 2, 2, 8, 128, 4, true, 2>(p, stream);
    case 3: return launch_tiled_layout<64, 64, 2, 2, 8, 64, 4, true, 2>(p, stream);
    default: return launch_big_layout_rowa(id, p, stream);
  }
}

}  // namespace dg
