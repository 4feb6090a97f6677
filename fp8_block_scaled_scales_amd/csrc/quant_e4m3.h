// Internal interface of the block quantiser kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

struct QuantArgs {
  const float* x;
  uint8_t* q;
  float* scales;
  int64_t rows, cols;
  int gran;
};

hipError_t launch_quant_e4m3(const QuantArgs& p, hipStream_t stream);

}  // namespace dg
