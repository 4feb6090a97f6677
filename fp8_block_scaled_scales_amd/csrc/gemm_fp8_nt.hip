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
//   * epilogue: FP32 -> BF16 round-to-nearest-even, staged through LDS so each
//     lane writes 16 contiguous bytes, masked at the M and N edges.
//
// Only this file and dg_host.hip make up the library; neither includes or
// calls any other code of the repository.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_fp8_nt.h"

namespace dg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int BK = 128;  // K bytes per pipeline step (row pitch of a staged slab)

// vmcnt(n) with expcnt and lgkmcnt left at their maxima (gfx9 encoding).
#define DG_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8))

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer (stride 0): any 16-byte access at offset >= bytes reads as zero.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Workgroup id -> (tile row, tile col).
// The dispatcher hands workgroup i to XCD i % 8. Renumber so that each XCD
// owns a contiguous run of the logical order, then walk that order as a
// grouped raster: GROUP_M tile rows advance together along N.
template <int GROUP_M>
__device__ __forceinline__ void map_tile(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  const int xcd = pid & 7, local = pid >> 3, q = nwg >> 3, r = nwg & 7;
  pid = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
  const int group = GROUP_M * tiles_n;
  const int gid = pid / group;
  const int first = gid * GROUP_M;
  const int gsz = min(tiles_m - first, GROUP_M);
  const int in = pid - gid * group;
  tm = first + in % gsz;
  tn = in / gsz;
}

// Copy a [ROWS x 128-byte] slab starting at column byte k0 of the rows the
// descriptor covers into LDS. One instruction per wave moves 8 rows (64 lanes
// x 16 B, written lane-contiguously from the wave-uniform LDS address). Lane
// L writes physical chunk L%8 of row L/8, so it fetches logical chunk
// (L%8) ^ (row%8): the XOR swizzle is applied on the global-address side.
template <int ROWS, int NWAVES>
__device__ __forceinline__ void stage_slab(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds, uint32_t K,
                                           uint32_t k0, int wave, int lane) {
  constexpr int GROUPS = ROWS / 8;
  static_assert(GROUPS % NWAVES == 0, "slab rows must split evenly over the waves");
  const uint32_t r_in = lane >> 3;
  const uint32_t chunk = (uint32_t)(lane & 7) ^ r_in;
#pragma unroll
  for (int i = 0; i < GROUPS / NWAVES; ++i) {
    const int grp = i * NWAVES + wave;
    const uint32_t row = grp * 8 + r_in;
    const uint32_t voff = row * K + k0 + chunk * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + grp * 1024), 16, voff, 0, 0, 0);
  }
}

// 32 bytes of K (logical 16-byte chunks c0 and c0+1) of one staged row.
__device__ __forceinline__ v8i frag32(const uint8_t* slab, int row, int c0) {
  const int sw = row & 7;
  const v4i lo = *reinterpret_cast<const v4i*>(slab + row * BK + ((c0 ^ sw) << 4));
  const v4i hi = *reinterpret_cast<const v4i*>(slab + row * BK + (((c0 + 1) ^ sw) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  // E4M3 x E4M3 (format code 0 for both operands), no block-exponent scaling.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // v_cvt_pk_bf16_f32: nearest even
}

template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M>
__global__ __launch_bounds__(64 * WM * WN) void gemm_fp8_nt_tiled(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ b, const float* __restrict__ sa,
    const float* __restrict__ sb, uint16_t* __restrict__ out, int M, int N, int K, int tiles_m,
    int tiles_n, int vec_store) {
  constexpr int NWAVES = WM * WN;
  constexpr int NT = 64 * NWAVES;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 sub-tiles per wave
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int SEGS = BK / G;      // K segments per pipeline step
  constexpr int KSTEPS = G / 64;    // MFMA K-steps per segment
  constexpr int LOADS = (BM / 8 + BN / 8) / NWAVES;  // buffer_load ... lds per wave per step
  constexpr int LDC = BN + 8;       // bf16 pitch of the epilogue tile (16-byte pad)
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 sub-tiles");
  static_assert(G % 32 == 0 && BK % G == 0, "granularity must cover whole sub-tiles and steps");
  static_assert(BM * LDC * 2 <= STAGES * STAGE_BYTES, "epilogue tile must fit in the ring");
  static_assert(LOADS < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  int tmi, tni;
  map_tile<GROUP_M>(tiles_m, tiles_n, tmi, tni);
  const int m0 = tmi * BM, n0 = tni * BN;
  const uint32_t uK = (uint32_t)K;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a + (int64_t)m0 * K, (uint32_t)min(BM, M - m0) * uK);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b + (int64_t)n0 * K, (uint32_t)min(BN, N - n0) * uK);

  const int nkb = K / G;                 // K segments
  const int nsteps = (K + BK - 1) / BK;  // pipeline steps

  // Scale rows of this wave's sub-tiles. A sub-tile lies inside one g-block
  // (g >= 32, sub-tiles aligned to 32); sub-tiles past the edge clamp to the
  // last block row so the index stays inside the scale tensor.
  const float* sa_row[TM];
  const float* sb_row[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) sa_row[t] = sa + (int64_t)min((m0 + wm * WTM + t * 32) / G, (M - 1) / G) * nkb;
#pragma unroll
  for (int t = 0; t < TN; ++t) sb_row[t] = sb + (int64_t)min((n0 + wn * WTN + t * 32) / G, (N - 1) / G) * nkb;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (v16f){};

  // Prologue: fill STAGES-1 ring slots.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    if (s < nsteps) {
      uint8_t* slot = smem + s * STAGE_BYTES;
      stage_slab<BM, NWAVES>(ra, slot, uK, s * BK, wave, lane);
      stage_slab<BN, NWAVES>(rb, slot + A_BYTES, uK, s * BK, wave, lane);
    }
  }

  const int arow = wm * WTM + (lane & 31);
  const int brow = wn * WTN + (lane & 31);
  const int half = lane >> 5;

  for (int s = 0; s < nsteps; ++s) {
    // Step s landed once only the later steps' loads are outstanding.
    if (STAGES == 3 && s + 1 < nsteps) {
      DG_WAIT_VMCNT(LOADS);
    } else {
      DG_WAIT_VMCNT(0);
    }
    __syncthreads();  // step s visible to all waves; slot (s-1)%STAGES free

    if (s + STAGES - 1 < nsteps) {
      const int sn = s + STAGES - 1;
      uint8_t* slot = smem + (sn % STAGES) * STAGE_BYTES;
      stage_slab<BM, NWAVES>(ra, slot, uK, sn * BK, wave, lane);
      stage_slab<BN, NWAVES>(rb, slot + A_BYTES, uK, sn * BK, wave, lane);
    }

    const uint8_t* As = smem + (s % STAGES) * STAGE_BYTES;
    const uint8_t* Bs = As + A_BYTES;
#pragma unroll
    for (int seg = 0; seg < SEGS; ++seg) {
      const int kb = s * SEGS + seg;
      if (kb >= nkb) break;  // K % 128 == 64 with g = 64: the last step holds one segment
      v8i af[TM][KSTEPS], bfr[TN][KSTEPS];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int c0 = (seg * KSTEPS + ks) * 4 + half * 2;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i][ks] = frag32(As, arow + i * 32, c0);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[j][ks] = frag32(Bs, brow + j * 32, c0);
      }
      float sbv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) sbv[j] = sb_row[j][kb];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const float sav = sa_row[i][kb];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v16f p = mfma_fp8(af[i][0], bfr[j][0], (v16f){});
#pragma unroll
          for (int ks = 1; ks < KSTEPS; ++ks) p = mfma_fp8(af[i][ks], bfr[j][ks], p);
          const float sc = sav * sbv[j];
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(p[v], sc, acc[i][j][v]);
        }
      }
    }
  }

  // Epilogue: BF16 tile through LDS, then 16-byte row-contiguous stores.
  __syncthreads();
  uint16_t* cs = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // 32x32 accumulator layout: lane%32 is the column, (v/4)*8 + (lane/32)*4 + v%4 the row.
        const int r = wm * WTM + i * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
        const int c = wn * WTN + j * 32 + (lane & 31);
        cs[r * LDC + c] = bf16_bits(acc[i][j][v]);
      }
  __syncthreads();
  constexpr int CHUNKS = BM * BN / 8;
  for (int idx = threadIdx.x; idx < CHUNKS; idx += NT) {
    const int r = idx / (BN / 8), c = (idx % (BN / 8)) * 8;
    const int gr = m0 + r, gc = n0 + c;
    if (gr >= M || gc >= N) continue;
    const v4i val = *reinterpret_cast<const v4i*>(cs + r * LDC + c);
    uint16_t* dst = out + (int64_t)gr * N + gc;
    if (vec_store && gc + 8 <= N) {
      *reinterpret_cast<v4i*>(dst) = val;
    } else {
      const uint16_t* e = reinterpret_cast<const uint16_t*>(&val);
      for (int t = 0; t < 8 && gc + t < N; ++t) dst[t] = e[t];
    }
  }
}

// ---- launch table -------------------------------------------------------------

template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M>
static hipError_t launch_tiled(const GemmArgs& p, hipStream_t stream) {
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_fp8_nt_tiled<BM, BN, WM, WN, STAGES, G, GROUP_M>), dim3(tiles_m * tiles_n),
                     dim3(64 * WM * WN), 0, stream, p.a, p.b, p.sa, p.sb, p.out, (int)p.M, (int)p.N,
                     (int)p.K, tiles_m, tiles_n, p.vec_store);
  return hipGetLastError();
}

KernelEntry kTable[] = {
    // id, bm, bn, stages, waves, ksplit, gran, launcher
    {0, 128, 128, 2, 4, 1, 128, &launch_tiled<128, 128, 2, 2, 2, 128, 4>},
    {1, 128, 128, 2, 4, 1, 64, &launch_tiled<128, 128, 2, 2, 2, 64, 4>},
};
const int kTableSize = sizeof(kTable) / sizeof(kTable[0]);

}  // namespace dg
