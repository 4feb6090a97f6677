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
  int gran;       // K segment of the kernel (64 or 128)
  int sshift;     // scale blocks are (gran << sshift) square: 1 for g = 256 on the gran-128 kernels
  int fmt;        // bit 0: A is E5M2 (else E4M3); bit 1: B is E5M2
  int rowa;       // A's factors are per row and K segment (1 x g blocks): sa is [M][K/g]
  int layout;     // bit 1: A stored [K,M]; bit 0: B stored [K,N] (0 = NT: A [M,K], B [N,K])
  int vec_store;  // out is 16-byte aligned and N % 8 == 0: full-row chunks use 16-byte stores
  int ksplit;     // workgroups per output tile along K (1 = no split)
  float* ws;      // split-K partial tiles, tiles * ksplit * bm * bn floats (ksplit > 1; caller's workspace)
  const float* bias;   // FP32 [N] added before the activation, or null
  int act;             // epilogue activation: 0 none, 1 ReLU, 2 GELU
};

typedef hipError_t (*Launcher)(const GemmArgs&, hipStream_t);

// Kernel classes of the tile table: 128x128 tiles over the whole K, small
// tiles whose K range is split over several workgroups (small M), 256-row
// tiles (256 or 128 columns) over the whole K (large M and N), and 32x32
// tiles over the whole K whose waves split K inside the workgroup (small M,
// many tiles).
enum TileClass { kClassTiled = 0, kClassSplitK = 1, kClassBig = 2, kClassStream = 3 };

// A table entry, with the constants of its launch-time estimate (see
// estimate_us in dg_host.hip): fixed costs per launch and per round of
// tiles, operand bytes and FLOP per second per CU, fitted to graph-timed
// launches of the entry over small to large shapes.
struct KernelEntry {
  int id;
  int cls;
  int bm, bn;
  int stages;
  int waves;
  int gran;
  Launcher launch;
  float launch_us;     // fixed cost per launch
  float round_us;      // fixed cost per round of one tile per CU
  float cu_gbps;       // operand bytes per CU per second, GB/s
  float cu_tflops;     // FLOP per CU per second, TFLOP/s
};

hipError_t launch_stream_g128(const GemmArgs& p, hipStream_t stream);
hipError_t launch_stream_g64(const GemmArgs& p, hipStream_t stream);
hipError_t launch_big_g128(const GemmArgs& p, hipStream_t stream);
hipError_t launch_big_g64(const GemmArgs& p, hipStream_t stream);
hipError_t launch_big128_g128(const GemmArgs& p, hipStream_t stream);
hipError_t launch_big128_g64(const GemmArgs& p, hipStream_t stream);

// The transposed layouts (GemmArgs::layout != 0) of table entry `id`: the
// tiled and split-K entries (0-3) and the 256- and 128-wide 256-row entries
// (4, 5, 9, 10); the _rowa forms take per-row A factors.
hipError_t launch_layout(int id, const GemmArgs& p, hipStream_t stream);
hipError_t launch_big_layout(int id, const GemmArgs& p, hipStream_t stream);
hipError_t launch_layout_rowa(int id, const GemmArgs& p, hipStream_t stream);
hipError_t launch_big_layout_rowa(int id, const GemmArgs& p, hipStream_t stream);

extern KernelEntry kTable[];
extern const int kTableSize;

}  // namespace dg
