// Block-scaled FP8 GEMM kernels for gfx950 (CDNA4, wave64).
//
// out[M,N] (BF16) = A[M,K] * B[N,K]^T with A, B in E4M3FN and one FP32 scale
// per g x g block of each operand (DeepGEMM实战 §2.2). Each g-wide K segment is
// contracted on the matrix cores into a fresh FP32 partial and then promoted
// into the running FP32 accumulator with one FMA by sa*sb (§2.2: scale
// handling fused into the main loop; §3.2: FP32 accumulation, K segments
// accumulated separately and then added).
//
// Structure of one workgroup (the generic tiled kernel):
//   * tile schedule: workgroup id -> output tile, remapped so that the tiles a
//     given XCD runs are contiguous in a grouped raster order, so concurrently
//     resident tiles on one XCD share A row panels and B column panels in that
//     XCD's L2 (the L2-locality point of the DeepGEMM-style template article,
//     §5.5);
//   * staging: each pipeline step moves a [BM x 128] slab of A and a
//     [BN x 128] slab of B from HBM straight into LDS with buffer_load ... lds
//     (16 bytes per lane), into a STAGES-deep ring (multi-buffering, template
//     article §3.3). Rows past M or N fall outside the buffer descriptor's
//     range and arrive as zeros (template article §5.5: zero the tile edge);
//     16-byte chunks are XOR-swizzled by row (template article §3.2) so the
//     fragment reads below are bank-conflict free;
//   * contraction: v_mfma_f32_32x32x64_f8f6f4, one 32x32 output sub-tile per
//     instruction, one (g=64) or two chained (g=128) instructions per segment
//     starting from a zero accumulator;
//   * promotion: acc = fma(partial, sa[mb,kb]*sb[nb,kb], acc), VALU, FP32;
//     with per-row A factors (one per row of A and K segment, the template
//     article's per-channel choice, §3.4) each step's factors for the tile's
//     rows are copied into LDS beside its slabs and the lane's sixteen row
//     factors replace sa[mb,kb];
//   * epilogue: FP32 -> BF16 round-to-nearest-even, staged through LDS so each
//     lane writes 16 contiguous bytes, masked at the M and N edges.
//
// The library is this directory's sources only; they include or call no other
// code of the repository.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "gemm_fp8_nt.h"
#include "gemm_fp8_tiled.h"

namespace dg {

KernelEntry kTable[] = {
    // id, class, bm, bn, stages, waves, gran, launcher,
    // estimate: us per launch, us per round, GB/s per CU, TFLOP/s per CU
    {0, kClassTiled, 128, 128, 2, 4, 128, &launch_tiled<128, 128, 2, 2, 2, 128, 4, false>, 6.0f, 0.0f, 54.0f, 7.0f},
    {1, kClassTiled, 128, 128, 2, 4, 64, &launch_tiled<128, 128, 2, 2, 2, 64, 4, false>, 6.0f, 0.0f, 40.0f, 5.5f},
    {2, kClassSplitK, 64, 64, 8, 4, 128, &launch_tiled<64, 64, 2, 2, 8, 128, 4, true>, 1.5f, 3.0f, 50.0f, 3.5f},
    {3, kClassSplitK, 64, 64, 8, 4, 64, &launch_tiled<64, 64, 2, 2, 8, 64, 4, true>, 1.5f, 3.0f, 38.0f, 2.5f},
    {4, kClassBig, 256, 256, 2, 8, 128, &launch_big_g128, 4.5f, 3.0f, 54.0f, 13.5f},
    {5, kClassBig, 256, 256, 2, 8, 64, &launch_big_g64, 4.5f, 3.0f, 42.0f, 10.5f},
    {6, kClassStream, 32, 32, 4, 4, 128, &launch_stream_g128, 2.5f, 2.0f, 70.0f, 2.5f},
    {7, kClassStream, 32, 32, 4, 4, 64, &launch_stream_g64, 1.5f, 3.0f, 64.0f, 2.5f},
    {9, kClassBig, 256, 128, 2, 8, 128, &launch_big128_g128, 1.5f, 3.0f, 56.0f, 10.0f},
    {10, kClassBig, 256, 128, 2, 8, 64, &launch_big128_g64, 2.5f, 3.0f, 48.0f, 8.0f},
};
const int kTableSize = sizeof(kTable) / sizeof(kTable[0]);

}  // namespace dg

