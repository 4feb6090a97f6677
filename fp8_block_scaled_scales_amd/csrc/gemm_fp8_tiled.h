// The tiled and split-K block-scaled FP8 GEMM kernel for gfx950 (template
// and launch helpers), shared by the NT table entries (gemm_fp8_nt.hip) and
// the transposed-operand layouts (gemm_fp8_layouts.hip). What the kernel
// computes and how is described at the top of gemm_fp8_nt.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "gemm_fp8_nt.h"

namespace dg {

constexpr int BK = 128;  // K bytes per pipeline step (row pitch of a staged slab)

// 32 bytes of K (logical 16-byte chunks c0 and c0+1) of one staged row. The
// slabs use the SW = 2 swizzle of stage_group: key (row % 8) ^ ((row / 8) % 2),
// so the rows one 16-byte read touches together hit distinct banks whether
// the read is served 8 lanes per clock or 16.
__device__ __forceinline__ v8i frag32(const uint8_t* slab, int row, int c0) {
  const int sw = (row & 7) ^ ((row >> 3) & 1);
  const v4i lo = *reinterpret_cast<const v4i*>(slab + row * BK + ((c0 ^ sw) << 4));
  const v4i hi = *reinterpret_cast<const v4i*>(slab + row * BK + (((c0 + 1) ^ sw) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// FMT bit 0: A is E5M2 (else E4M3), bit 1: B is E5M2 -- the instruction's
// operand-format fields (0 = E4M3, 1 = E5M2); no block-exponent scaling.
template <int FMT>
__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT & 1, FMT >> 1, 0, 0, 0, 0);
}

// Wait until at most `steps` later pipeline steps' loads (LOADS each) are
// still in flight for this wave; steps is 0 .. MAXS.
template <int LOADS, int MAXS>
__device__ __forceinline__ void wait_steps(int steps) {
  if constexpr (MAXS == 0) {
    DG_WAIT_VMCNT(0);
  } else {
    if (steps >= MAXS) {
      DG_WAIT_VMCNT(LOADS * MAXS);
    } else {
      wait_steps<LOADS, MAXS - 1>(steps);
    }
  }
}

// Split-K: ksplit workgroups share one output tile, each covering a contiguous
// range of 128-byte K steps, and each writes its FP32 partial tile to ws (the
// caller's workspace) with plain stores. A second kernel on the same stream,
// splitk_reduce, adds the partials in split order (so the result does not
// depend on which split ran when) and writes the BF16 tile with the
// epilogue: the kernel boundary orders the two, so no workgroup waits for or
// signals another and nothing in the workspace is read before this call
// wrote it. ksplit == 1 skips all of this.
//
// G is the K segment contracted before each promotion; the scale blocks are
// sg x sg with sg = G << sshift (g = 256 runs G = 128 with one factor per two
// segments). ROWA: A's factors are per row, sa is [M][K/sg]. LAYOUT bit 1: A
// stored [K,M]; bit 0: B stored [K,N] (M resp. N any length).
template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M, bool SPLIT, int FMT, int EPI, bool ROWA,
          int LAYOUT>
__global__ __launch_bounds__(64 * WM * WN) void gemm_fp8_nt_tiled(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ b, const float* __restrict__ sa,
    const float* __restrict__ sb, uint16_t* __restrict__ out, int M, int N, int K, int tiles_m,
    int tiles_n, int vec_store, int ksplit, float* __restrict__ ws, int sshift, const float* __restrict__ bias,
    int relu) {
  constexpr int NWAVES = WM * WN;
  constexpr int NT = 64 * NWAVES;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 sub-tiles per wave
  constexpr int SEGS = BK / G;      // K segments per pipeline step
  constexpr int KSTEPS = G / 64;    // MFMA K-steps per segment
  constexpr int SCL = ROWA ? NWAVES * 256 : 0;  // per-row factors of a step: [SEGS][BM] FP32, a piece per wave
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, STAGE_BYTES = A_BYTES + B_BYTES + SCL;
  // buffer_load ... lds per wave per step (the factor piece included)
  constexpr int LOADS = (BM / 8 + BN / 8) / NWAVES + (ROWA ? 1 : 0);
  constexpr int LDC = BN + 8;       // bf16 pitch of the epilogue tile (16-byte pad)
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 sub-tiles");
  static_assert(G % 32 == 0 && BK % G == 0, "granularity must cover whole sub-tiles and steps");
  static_assert(BM * LDC * 2 <= STAGES * STAGE_BYTES, "epilogue tile must fit in the ring");
  static_assert(LOADS * (STAGES - 2) < 64, "vmcnt range");
  static_assert(BM * SEGS <= NWAVES * 64, "a step's row factors: one 64-entry piece per wave");

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

  const int nkb = K / G;                       // K segments
  const int nsteps_all = (K + BK - 1) / BK;    // pipeline steps over the whole K
  const int st0 = (int)((int64_t)ks * nsteps_all / ksplit);
  const int nsteps = (int)((int64_t)(ks + 1) * nsteps_all / ksplit) - st0;  // this split's steps

  // Scale rows of this wave's sub-tiles. A sub-tile lies inside one g-block
  // (g >= 32, sub-tiles aligned to 32); sub-tiles past the edge clamp to the
  // last block row so the index stays inside the scale tensor.
  const int sg = G << sshift, nks = K / sg;  // scale blocks
  const v4i rsa = ROWA ? rsrc_words(sa + (int64_t)m0 * nks, (uint32_t)min(BM, M - m0) * (uint32_t)nks * 4u) : (v4i){};
  auto stage_step = [&](int s) {  // the copies of this split's step s into its ring slot
    uint8_t* slot = smem + (s % STAGES) * STAGE_BYTES;
    const int st = st0 + s;
    if constexpr (ROWA)
      stage_row_scales<BM, SEGS>(rsa, slot + A_BYTES + B_BYTES, (uint32_t)nks, (uint32_t)((st * SEGS) >> sshift), wave,
                                 lane);
    const int64_t k0 = (int64_t)st * BK;
    if constexpr ((LAYOUT & 2) != 0) {
      // the step's K rows of A^T from column m0; past the tensor reads zero
      const v4i rat = rsrc_words(a + k0 * M + m0, tile_range_t(k0, K, M, m0, BK));
#pragma unroll
      for (int i = 0; i < BM / 8 / NWAVES; ++i) stage_group_t<BM>(rat, slot, (uint32_t)M, i * NWAVES + wave, lane);
    } else {
      stage_slab<BM, NWAVES, 2>(ra, slot, uK, st * BK, wave, lane);
    }
    if constexpr ((LAYOUT & 1) != 0) {
      const v4i rbt = rsrc_words(b + k0 * N + n0, tile_range_t(k0, K, N, n0, BK));
#pragma unroll
      for (int i = 0; i < BN / 8 / NWAVES; ++i)
        stage_group_t<BN>(rbt, slot + A_BYTES, (uint32_t)N, i * NWAVES + wave, lane);
    } else {
      stage_slab<BN, NWAVES, 2>(rb, slot + A_BYTES, uK, st * BK, wave, lane);
    }
  };
  const float* sa_row[TM];
  const float* sb_row[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) sa_row[t] = sa + (int64_t)min((m0 + wm * WTM + t * 32) / sg, (M - 1) / sg) * nks;
#pragma unroll
  for (int t = 0; t < TN; ++t) sb_row[t] = sb + (int64_t)min((n0 + wn * WTN + t * 32) / sg, (N - 1) / sg) * nks;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (v16f){};

  // The epilogue's bias for this lane's columns, loaded before the first
  // copies: the step waits cover it, and no output store is in flight when
  // the epilogue reads it.
  const bool hb = EPI != 0 && bias != nullptr;
  float bcol[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * WTN + j * 32 + (lane & 31);
    bcol[j] = hb && col < N ? bias[col] : 0.0f;
  }

  // Prologue: fill STAGES-1 ring slots.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nsteps) stage_step(s);

  const int arow = wm * WTM + (lane & 31);
  const int brow = wn * WTN + (lane & 31);
  const int half = lane >> 5;

  for (int s = 0; s < nsteps; ++s) {
    // Step s landed once only the later steps' loads are outstanding.
    wait_steps<LOADS, STAGES - 2>(min(STAGES - 2, nsteps - 1 - s));
    __syncthreads();  // step s visible to all waves; slot (s-1)%STAGES free
    if constexpr (LAYOUT != 0) {
      // the tensor's last K row of a transposed operand whose stored row
      // length is not a multiple of 4 (see patch_tail_t)
      if (st0 + s == nsteps_all - 1 && (((LAYOUT & 2) && (M & 3)) || ((LAYOUT & 1) && (N & 3)))) {
        if (wave == 0) {
          uint8_t* slot = smem + (s % STAGES) * STAGE_BYTES;
          const int64_t k0 = (int64_t)(st0 + s) * BK;
          if ((LAYOUT & 2) && (M & 3)) patch_tail_t<BM>(slot, a, (int64_t)K * M, M, k0, m0, lane);
          if ((LAYOUT & 1) && (N & 3)) patch_tail_t<BN>(slot + A_BYTES, b, (int64_t)K * N, N, k0, n0, lane);
        }
        __syncthreads();
      }
    }

    if (s + STAGES - 1 < nsteps) stage_step(s + STAGES - 1);

    const uint8_t* As = smem + (s % STAGES) * STAGE_BYTES;
    const uint8_t* Bs = As + A_BYTES;
    // ROWA: the step's factors [SEGS][BM]; this lane's rows of sub-tile i are
    // wm*WTM + 32i + 8c + 4*half .. +3
    const float* const scl = reinterpret_cast<const float*>(As + A_BYTES + B_BYTES) + wm * WTM + 4 * half;
#pragma unroll
    for (int seg = 0; seg < SEGS; ++seg) {
      const int kb = (st0 + s) * SEGS + seg;
      if (kb >= nkb) break;  // K % 128 == 64 with g = 64: the last step holds one segment
      v8i af[TM][KSTEPS], bfr[TN][KSTEPS];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int c0 = (seg * KSTEPS + ks) * 4 + half * 2;
        const int kofs = (seg * KSTEPS + ks) * 64;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if constexpr ((LAYOUT & 2) != 0) {
            af[i][ks] = frag_tr<BM>(As, wm * WTM + i * 32, kofs, lane);
          } else {
            af[i][ks] = frag32(As, arow + i * 32, c0);
          }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr ((LAYOUT & 1) != 0) {
            bfr[j][ks] = frag_tr<BN>(Bs, wn * WTN + j * 32, kofs, lane);
          } else {
            bfr[j][ks] = frag32(Bs, brow + j * 32, c0);
          }
        }
      }
      float sbv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) sbv[j] = sb_row[j][kb >> sshift];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const float sav = ROWA ? 0.0f : sa_row[i][kb >> sshift];
        v4f sr[4];
        if constexpr (ROWA) {
#pragma unroll
          for (int c = 0; c < 4; ++c) sr[c] = *reinterpret_cast<const v4f*>(scl + seg * BM + i * 32 + 8 * c);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v16f p = mfma_fp8<FMT>(af[i][0], bfr[j][0], (v16f){});
#pragma unroll
          for (int ks = 1; ks < KSTEPS; ++ks) p = mfma_fp8<FMT>(af[i][ks], bfr[j][ks], p);
          if constexpr (ROWA) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(p[v], sr[v >> 2][v & 3] * sbv[j], acc[i][j][v]);
          } else {
            const float sc = sav * sbv[j];
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(p[v], sc, acc[i][j][v]);
          }
        }
      }
    }
    DG_STEP_SYNC_WG();
  }

  if (SPLIT && ksplit > 1) {
    // This split's FP32 partial tile, row-major, to its slot of the
    // workspace; splitk_reduce (launched next on the same stream) adds the
    // splits and writes the output. Each store covers two tile rows of 32
    // columns (128 contiguous bytes each).
    float* part = ws + ((int64_t)(tmi * tiles_n + tni) * ksplit + ks) * (BM * BN);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WTM + i * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
          const int c = wn * WTN + j * 32 + (lane & 31);
          part[r * BN + c] = acc[i][j][v];
        }
    return;
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
        cs[r * LDC + c] = bf16_bits(epilogue_fn<EPI>(acc[i][j][v], hb, bcol[j], relu));
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
      for (int t = 0; t < 8 && gc + t < N; ++t) dst[t] = (uint16_t)((uint32_t)val[t >> 1] >> (16 * (t & 1)));
    }
  }
}

// Second kernel of a K split: out = epilogue(sum over splits 0, 1, ...,
// ksplit-1 of the partial tiles), the additions in split order, in FP32, then
// rounded to BF16. One thread per four consecutive columns of a tile row; the
// grid covers every tile (tiles * BM * BN / 4 threads, 256 per workgroup),
// and threads past M or N store nothing.
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ ws, uint16_t* __restrict__ out, int M,
                                                     int N, int tiles_n, int ksplit, int vec_store,
                                                     const float* __restrict__ bias, int relu) {
  constexpr int Q = BN / 4;  // float4 per tile row
  static_assert((BM * Q) % 256 == 0, "whole workgroups per tile");
  const int tile = (int)(blockIdx.x / ((BM * Q) / 256));
  const int e = (int)(blockIdx.x % ((BM * Q) / 256)) * 256 + (int)threadIdx.x;
  const int r = e / Q, c = (e % Q) * 4;
  const int gr = (tile / tiles_n) * BM + r, gc = (tile % tiles_n) * BN + c;
  if (gr >= M || gc >= N) return;
  const float* p = ws + (int64_t)tile * ksplit * (BM * BN) + r * BN + c;
  v4f sum = {0.0f, 0.0f, 0.0f, 0.0f};
  int sp = 0;
  for (; sp + 8 <= ksplit; sp += 8) {  // eight loads in flight, added in order
    v4f q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = *reinterpret_cast<const v4f*>(p + (int64_t)(sp + t) * (BM * BN));
#pragma unroll
    for (int t = 0; t < 8; ++t) sum += q[t];
  }
  for (; sp < ksplit; ++sp) sum += *reinterpret_cast<const v4f*>(p + (int64_t)sp * (BM * BN));
  const bool hb = EPI != 0 && bias != nullptr;
  uint16_t h[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) h[t] = bf16_bits(epilogue_fn<EPI>(sum[t], hb, hb && gc + t < N ? bias[gc + t] : 0.0f, relu));
  uint16_t* dst = out + (int64_t)gr * N + gc;
  if (vec_store && gc + 4 <= N) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
  } else {
    for (int t = 0; t < 4 && gc + t < N; ++t) dst[t] = h[t];
  }
}

// ---- launch table -------------------------------------------------------------

template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M, bool SPLIT, int FMT, int EPI, bool ROWA,
          int LAYOUT>
static hipError_t launch_tiled_fa(const GemmArgs& p, hipStream_t stream) {
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_fp8_nt_tiled<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, FMT, EPI, ROWA, LAYOUT>),
                     dim3(tiles_m * tiles_n * p.ksplit), dim3(64 * WM * WN), 0, stream, p.a, p.b, p.sa, p.sb, p.out,
                     (int)p.M, (int)p.N, (int)p.K, tiles_m, tiles_n, p.vec_store, p.ksplit, p.ws, p.sshift, p.bias,
                     p.act == 1 ? 1 : 0);
  hipError_t err = hipGetLastError();
  if (SPLIT && p.ksplit > 1 && err == hipSuccess) {
    hipLaunchKernelGGL((splitk_reduce<BM, BN, EPI>), dim3(tiles_m * tiles_n * (BM * BN / 4 / 256)), dim3(256), 0,
                       stream, p.ws, p.out, (int)p.M, (int)p.N, tiles_n, p.ksplit, p.vec_store, p.bias,
                       p.act == 1 ? 1 : 0);
    err = hipGetLastError();
  }
  return err;
}

// RS selects the A factor forms compiled: 0 both, chosen by p.rowa (the NT
// entries); 1 g x g blocks only; 2 per-row factors only (the transposed
// layouts compile the two forms in separate translation units).
template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M, bool SPLIT, int FMT, int EPI, int LAYOUT,
          int RS>
static hipError_t launch_tiled_sa(const GemmArgs& p, hipStream_t stream) {
  if constexpr (RS == 1) {
    return p.rowa ? hipErrorInvalidValue
                  : launch_tiled_fa<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, FMT, EPI, false, LAYOUT>(p, stream);
  } else if constexpr (RS == 2) {
    return p.rowa ? launch_tiled_fa<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, FMT, EPI, true, LAYOUT>(p, stream)
                  : hipErrorInvalidValue;
  } else {
    return p.rowa ? launch_tiled_fa<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, FMT, EPI, true, LAYOUT>(p, stream)
                  : launch_tiled_fa<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, FMT, EPI, false, LAYOUT>(p, stream);
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M, bool SPLIT, int FMT, int LAYOUT, int RS>
static hipError_t launch_tiled_fmt(const GemmArgs& p, hipStream_t stream) {
  switch (epilogue_form(p.bias, p.act)) {
    case 0: return launch_tiled_sa<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, FMT, 0, LAYOUT, RS>(p, stream);
    case 1: return launch_tiled_sa<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, FMT, 1, LAYOUT, RS>(p, stream);
    case 2: return launch_tiled_sa<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, FMT, 2, LAYOUT, RS>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M, bool SPLIT, int LAYOUT, int RS>
static hipError_t launch_tiled_l(const GemmArgs& p, hipStream_t stream) {
  if ((!SPLIT && p.ksplit != 1) || p.sshift < 0 || p.sshift > 1) return hipErrorInvalidValue;
  switch (p.fmt) {
    case 0: return launch_tiled_fmt<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, 0, LAYOUT, RS>(p, stream);
    case 1: return launch_tiled_fmt<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, 1, LAYOUT, RS>(p, stream);
    case 2: return launch_tiled_fmt<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, 2, LAYOUT, RS>(p, stream);
    case 3: return launch_tiled_fmt<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, 3, LAYOUT, RS>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// The NT table entries.
template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M, bool SPLIT>
static hipError_t launch_tiled(const GemmArgs& p, hipStream_t stream) {
  return p.layout == 0 ? launch_tiled_l<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, 0, 0>(p, stream)
                       : hipErrorInvalidValue;
}

// The transposed layouts on the same tile, with the A factor form RS
// (instantiated in gemm_fp8_layouts.hip and gemm_fp8_layouts_rowa.hip).
template <int BM, int BN, int WM, int WN, int STAGES, int G, int GROUP_M, bool SPLIT, int RS>
static hipError_t launch_tiled_layout(const GemmArgs& p, hipStream_t stream) {
  switch (p.layout) {
    case 1: return launch_tiled_l<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, 1, RS>(p, stream);
    case 2: return launch_tiled_l<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, 2, RS>(p, stream);
    case 3: return launch_tiled_l<BM, BN, WM, WN, STAGES, G, GROUP_M, SPLIT, 3, RS>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
