// Large-tile block-scaled FP8 GEMM for gfx950: 256 x 256 output tiles.
//
// Same operation as the other kernels (DeepGEMM实战 §2.2: one FP32 scale per
// g x g block of each operand, restored while the products are accumulated,
// the scale handling fused into the main loop; §3.2: FP32 accumulation, each
// K segment summed on its own and the segments then added; §3.3/§4.2: NT
// layout, A [M,K] and B [N,K] K-contiguous, BF16 out).
//
// Why this shape. On MI355X a CU's L2->LDS intake is about 50 bytes per clock
// and its FP8 matrix rate 8192 FLOP per clock, so a tile must do at least
// ~170 FLOPs per staged byte to keep the matrix cores fed: 2*BM*BN/(BM+BN) is
// 128 for 128x128 and 256 for 256x256. A 256x256x128 step stages 64 KB and
// does 16.8 MFLOP (2048 clocks at peak); two ring slots fill 128 KB of the
// 160 KB LDS.
//
// Workgroup: 8 waves (two per SIMD), laid out 2 (M) x 4 (N), each owning a
// 128 x 64 sub-tile with its FP32 accumulator in 128 VGPRs. Per 128-byte K
// step:
//   * g = 128: the step is one K segment. Each 16 x 16 output block is one
//     v_mfma_f32_16x16x128_f8f6f4 from a zero accumulator (the whole segment
//     in one instruction), promoted with acc = fma(partial, sa*sb, acc);
//   * g = 64: the step holds two segments. Each 32 x 32 output block per
//     segment is one v_mfma_f32_32x32x64_f8f6f4 from zero, promoted the same
//     way; the wave's 128 rows span two row blocks of scales.
// The tiles' LDS slabs use the SW = 1 swizzle: the 16 (or 32) rows a fragment
// read touches together hit distinct banks.
//
// Epilogue: the BF16 tile goes through LDS in two 128-row halves so every
// lane stores 16 contiguous bytes, masked at the M and N edges.
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
#include "gemm_fp8_nt.h"

namespace dg {

namespace big {

constexpr int BM = 256, BN = 256, BK = 128, STAGES = 2;
constexpr int WM = 2, WN = 4, NW = WM * WN, NT = 64 * NW;
constexpr int WTM = BM / WM, WTN = BN / WN;  // 128 x 64 wave tile
constexpr int A_BYTES = BM * BK, STAGE_BYTES = (BM + BN) * BK;
constexpr int LOADS = (BM / 8 + BN / 8) / NW;  // HBM->LDS instructions per wave per step
constexpr int LDC = BN + 8;                    // bf16 pitch of the epilogue half-tile
static_assert(WTM * LDC * 2 <= STAGES * STAGE_BYTES, "epilogue half-tile must fit in the ring");

// 32 K bytes (logical 16-byte chunks c0, c0+1) of staged row `row` under the
// SW = 1 swizzle.
__device__ __forceinline__ v8i frag(const uint8_t* slab, int row, int c0) {
  const int sw = (row >> 1) & 7;
  const v4i lo = *reinterpret_cast<const v4i*>(slab + row * BK + ((c0 ^ sw) << 4));
  const v4i hi = *reinterpret_cast<const v4i*>(slab + row * BK + (((c0 + 1) ^ sw) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

__device__ __forceinline__ v4f mfma16(const v8i& a, const v8i& b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, (v4f){}, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma32(const v8i& a, const v8i& b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, (v16f){}, 0, 0, 0, 0, 0, 0);
}

// Accumulator: 128 FP32 per lane either way.
template <int G>
struct Acc;
template <>
struct Acc<128> {
  v4f t[WTM / 16][WTN / 16];  // 8 x 4 blocks of 16 x 16
};
template <>
struct Acc<64> {
  v16f t[WTM / 32][WTN / 32];  // 4 x 2 blocks of 32 x 32
};

template <int G, int GROUP_M>
__global__ __launch_bounds__(NT) void gemm_fp8_nt_big(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                      const float* __restrict__ sa, const float* __restrict__ sb,
                                                      uint16_t* __restrict__ out, int M, int N, int K, int tiles_m,
                                                      int tiles_n, int vec_store) {
  static_assert(G == 64 || G == 128, "granularity");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  int ks, tmi, tni;
  map_tile<GROUP_M>(tiles_m, tiles_n, ks, tmi, tni);
  const int m0 = tmi * BM, n0 = tni * BN;
  const uint32_t uK = (uint32_t)K;
  const v4i ra = rsrc_words(a + (int64_t)m0 * K, (uint32_t)min(BM, M - m0) * uK);
  const v4i rb = rsrc_words(b + (int64_t)n0 * K, (uint32_t)min(BN, N - n0) * uK);

  const int nkb = K / G;
  const int nsteps = (K + BK - 1) / BK;

  // Scale rows of this wave. Rows of a block past the edge clamp to the last
  // block row (their data is zero).
  const int wr0 = m0 + wm * WTM, wc0 = n0 + wn * WTN;
  const float* const sa0 = sa + (int64_t)min(wr0 / G, (M - 1) / G) * nkb;
  const float* const sa1 = sa + (int64_t)min((wr0 + 64) / G, (M - 1) / G) * nkb;  // g = 64: second row block
  const float* const sbr = sb + (int64_t)min(wc0 / G, (N - 1) / G) * nkb;

  Acc<G> acc;
  if constexpr (G == 128) {
#pragma unroll
    for (int i = 0; i < WTM / 16; ++i)
#pragma unroll
      for (int j = 0; j < WTN / 16; ++j) acc.t[i][j] = (v4f){};
  } else {
#pragma unroll
    for (int i = 0; i < WTM / 32; ++i)
#pragma unroll
      for (int j = 0; j < WTN / 32; ++j) acc.t[i][j] = (v16f){};
  }

  stage_slab<BM, NW, 1>(ra, smem, uK, 0, wave, lane);
  stage_slab<BN, NW, 1>(rb, smem + A_BYTES, uK, 0, wave, lane);

  for (int s = 0; s < nsteps; ++s) {
    DG_WAIT_VMCNT(0);  // this wave's part of step s has landed
    __syncthreads();   // all of step s visible; the other slot is free
    if (s + 1 < nsteps) {
      uint8_t* slot = smem + ((s + 1) & 1) * STAGE_BYTES;
      stage_slab<BM, NW, 1>(ra, slot, uK, (s + 1) * BK, wave, lane);
      stage_slab<BN, NW, 1>(rb, slot + A_BYTES, uK, (s + 1) * BK, wave, lane);
    }
    const uint8_t* As = smem + (s & 1) * STAGE_BYTES + wm * WTM * BK;
    const uint8_t* Bs = smem + (s & 1) * STAGE_BYTES + A_BYTES + wn * WTN * BK;

    if constexpr (G == 128) {
      const int r16 = lane & 15, q = lane >> 4;
      const float sc = sa0[s] * sbr[s];
      v8i bf[WTN / 16];
#pragma unroll
      for (int j = 0; j < WTN / 16; ++j) bf[j] = frag(Bs, j * 16 + r16, 2 * q);
#pragma unroll
      for (int i = 0; i < WTM / 16; ++i) {
        const v8i af = frag(As, i * 16 + r16, 2 * q);
#pragma unroll
        for (int j = 0; j < WTN / 16; ++j) {
          const v4f p = mfma16(af, bf[j]);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc.t[i][j][v] = __builtin_fmaf(p[v], sc, acc.t[i][j][v]);
        }
      }
    } else {
      const int r32 = lane & 31, h2 = lane >> 5;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = 2 * s + h;
        if (kb < nkb) {  // K % 128 == 64: the last step holds one segment
          const float sbv = sbr[kb];
          const float sc0 = sa0[kb] * sbv, sc1 = sa1[kb] * sbv;
          v8i bf[WTN / 32];
#pragma unroll
          for (int j = 0; j < WTN / 32; ++j) bf[j] = frag(Bs, j * 32 + r32, 4 * h + 2 * h2);
#pragma unroll
          for (int i = 0; i < WTM / 32; ++i) {
            const v8i af = frag(As, i * 32 + r32, 4 * h + 2 * h2);
            const float sc = i < 2 ? sc0 : sc1;
#pragma unroll
            for (int j = 0; j < WTN / 32; ++j) {
              const v16f p = mfma32(af, bf[j]);
#pragma unroll
              for (int v = 0; v < 16; ++v) acc.t[i][j][v] = __builtin_fmaf(p[v], sc, acc.t[i][j][v]);
            }
          }
        }
      }
    }
  }

  // Epilogue, two halves of 128 rows: the waves of wave-row `half` write
  // their BF16 sub-tiles to LDS, then all threads store the half.
  uint16_t* cs = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int half = 0; half < WM; ++half) {
    __syncthreads();
    if (wm == half) {
      if constexpr (G == 128) {
        const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
        for (int i = 0; i < WTM / 16; ++i)
#pragma unroll
          for (int j = 0; j < WTN / 16; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              cs[(i * 16 + 4 * q + v) * LDC + wn * WTN + j * 16 + r16] = bf16_bits(acc.t[i][j][v]);
      } else {
        const int r32 = lane & 31, h2 = lane >> 5;
#pragma unroll
        for (int i = 0; i < WTM / 32; ++i)
#pragma unroll
          for (int j = 0; j < WTN / 32; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              cs[(i * 32 + 8 * (v >> 2) + 4 * h2 + (v & 3)) * LDC + wn * WTN + j * 32 + r32] =
                  bf16_bits(acc.t[i][j][v]);
      }
    }
    __syncthreads();
    constexpr int CHUNKS = WTM * BN / 8;
#pragma unroll
    for (int it = 0; it < CHUNKS / NT; ++it) {
      const int idx = it * NT + threadIdx.x;
      const int r = idx / (BN / 8), c = (idx % (BN / 8)) * 8;
      const int gr = m0 + half * WTM + r, gc = n0 + c;
      if (gr >= M || gc >= N) continue;
      const v4i val = *reinterpret_cast<const v4i*>(cs + r * LDC + c);
      uint16_t* dst = out + (int64_t)gr * N + gc;
      if (vec_store && gc + 8 <= N) {
        *reinterpret_cast<v4i*>(dst) = val;
      } else {
        for (int t = 0; t < 8 && gc + t < N; ++t) dst[t] = (uint16_t)((uint32_t)val[t >> 1] >> (16 * (t & 1)));
      }
    }
  }
}

template <int G, int GROUP_M>
hipError_t launch(const GemmArgs& p, hipStream_t stream) {
  if (p.ksplit != 1) return hipErrorInvalidValue;
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_fp8_nt_big<G, GROUP_M>), dim3(tiles_m * tiles_n), dim3(NT), 0, stream, p.a, p.b, p.sa, p.sb,
                     p.out, (int)p.M, (int)p.N, (int)p.K, tiles_m, tiles_n, p.vec_store);
  return hipGetLastError();
}

}  // namespace big

hipError_t launch_big_g128(const GemmArgs& p, hipStream_t s) { return big::launch<128, 4>(p, s); }
hipError_t launch_big_g64(const GemmArgs& p, hipStream_t s) { return big::launch<64, 4>(p, s); }

}  // namespace dg
