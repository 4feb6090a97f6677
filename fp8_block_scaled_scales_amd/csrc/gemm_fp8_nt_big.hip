// The NT table entries of the 256-row-tile kernel (gemm_fp8_big.h), 256 and
// 128 columns wide at g = 128 and 64: a translation unit of their own so these
// heavy instances compile beside the others.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "gemm_fp8_big.h"
#include "gemm_fp8_nt.h"

namespace dg {

hipError_t launch_big_g128(const GemmArgs& p, hipStream_t s) { return big::launch<128, 256, 2>(p, s); }
hipError_t launch_big_g64(const GemmArgs& p, hipStream_t s) { return big::launch<64, 256, 2>(p, s); }
hipError_t launch_big128_g128(const GemmArgs& p, hipStream_t s) { return big::launch<128, 128, 4>(p, s); }
hipError_t launch_big128_g64(const GemmArgs& p, hipStream_t s) { return big::launch<64, 128, 4>(p, s); }

}  // namespace dg

