// Large-tile block-scaled FP8 GEMM for gfx950: 256 x BN output tiles,
// BN = 256 or 128.
//
// Same operation as the other kernels (DeepGEMM实战 §2.2: one FP32 scale per
// g x g block of each operand, restored while the products are accumulated,
// the scale handling fused into the main loop; §3.2: FP32 accumulation, each
// K segment summed on its own and the segments then added; §3.3/§4.2: NT
// layout, A [M,K] and B [N,K] K-contiguous, BF16 out).
//
// Why this shape. On MI355X a CU's L2->LDS intake is about 50-70 bytes per
// clock and its FP8 matrix rate 8192 FLOP per clock, so a tile must do at
// least ~170 FLOPs per staged byte to keep the matrix cores fed: 2*BM*BN/(BM+BN)
// is 128 for 128x128 and 256 for 256x256. A 256x256x128 step stages 64 KB and
// does 16.8 MFLOP (2048 clocks at peak); two ring slots fill 128 KB of the
// 160 KB LDS. The narrower tile exists for tile counts: 256x128 gives a
// 2000 x 4000 output 256 tiles, one per CU, where 256x256 would leave half the
// chip idle. (A 256x224 tile, which splits a 7168-wide N into 32 tiles, was
// measured slower per step than 256x256, so never worth its better fill.)
//
// Workgroup: 8 waves (two per SIMD), laid out WM x WN, each owning a
// WTM x WTN sub-tile with its FP32 accumulator in registers. Per 128-byte K
// step:
//   * g = 128: the step is one K segment. Each 16 x 16 output block is one
//     v_mfma_f32_16x16x128_f8f6f4 from a zero accumulator (the whole segment
//     in one instruction), promoted with acc = fma(partial, sa*sb, acc);
//   * g = 64: the step holds two segments. Each 32 x 32 output block per
//     segment is one v_mfma_f32_32x32x64_f8f6f4 from zero, promoted the same
//     way; a 128-row wave tile spans two row blocks of scales.
// Instruction order inside a step is fixed by hand (schedule barriers): the
// MFMAs go out back to back and each promotion runs a few MFMAs behind its
// own, so the matrix core never waits for the FMA of the block it just
// produced; A fragments are read from LDS one row block ahead.
// The next step's copies are issued by waves 0-3 at the start of the step and
// by waves 4-7 a quarter of the way in: the memory pipeline takes one 1 KB
// copy per ~14 clocks and a wave stalls until its copy is taken, so this way
// one wave per SIMD is always free to issue MFMAs.
// The tiles' LDS slabs use the SW = 2 swizzle: the 16 (or 32) rows a fragment
// read touches together hit distinct banks.
//
// Epilogue: the BF16 tile goes through LDS in two 128-row passes so every
// lane stores 16 contiguous bytes, masked at the M and N edges.
//
// Per-row A factors (ROWA; one factor per row of A and K segment, the
// template article's per-channel choice, §3.4): each step's factors for the
// tile's 256 rows are copied with the step's slabs into a 2 KB area after
// them (one 4-byte-per-lane copy per wave), and a promotion multiplies the
// lane's four (16x16 layout) or sixteen (32x32 layout) row factors by the
// column block's factor in place of the one block product.
//
// MFMA layouts used. 16x16x128: lane l supplies row (A) or column (B) l%16
// and 32 K bytes starting at 32*(l/16); result register v of lane l is row
// 4*(l/16)+v, column l%16. 32x32x64: lane l supplies row/column l%32 and 32 K
// bytes starting at 32*(l/32); result register v is row
// 8*(v/4) + 4*(l/32) + v%4, column l%32. A and B fragments are loaded the same
// way, so every A byte meets the B byte of the same K.
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

