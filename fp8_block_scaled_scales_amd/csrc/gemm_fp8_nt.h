// Internal interface between the host dispatcher and the kernel table.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  uint16_t* out;
  int64_t M, N, K;
  int gran;
  int vec_store;  // out is 16-byte aligned and N % 8 == 0: full-row chunks use 16-byte stores
};

typedef hipError_t (*Launcher)(const GemmArgs&, hipStream_t);

struct KernelEntry {
  int id;
  int bm, bn;
  int stages;
  int waves;
  int ksplit;
  int gran;
  Launcher launch;
};

extern KernelEntry kTable[];
extern const int kTableSize;

}  // namespace dg
