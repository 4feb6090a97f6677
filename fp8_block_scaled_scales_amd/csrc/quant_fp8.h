// Internal interface of the block quantiser kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

struct QuantArgs {
  const void* x;  // [rows][cols] elements of kind `in`
  uint8_t* q;
  float* scales;
  int64_t rows, cols;
  int gran;  // 64, 128 or 256
  int fmt;   // 0 = E4M3FN, 1 = E5M2
  int in;    // input elements: 0 = FP32, 1 = BF16, 2 = FP16
};

hipError_t launch_quant(const QuantArgs& p, hipStream_t stream);       // g x g blocks: scales [ceil(rows/g)][cols/g]
hipError_t launch_quant_rows(const QuantArgs& p, hipStream_t stream);  // 1 x g blocks: scales [rows][cols/g]

}  // namespace dg
