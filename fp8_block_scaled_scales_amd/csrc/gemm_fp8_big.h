// The 256-row-tile block-scaled FP8 GEMM kernel for gfx950 (template and
// launch helpers), instantiated for the NT table entries
// (gemm_fp8_nt_big.hip) and the transposed-operand layouts
// (gemm_fp8_big_layouts.hip, gemm_fp8_big_layouts_rowa.hip).
//
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
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "gemm_fp8_nt.h"

namespace dg {

namespace big {

constexpr int BM = 256, BK = 128, NW = 8, NT = 64 * NW;
constexpr int A_BYTES = BM * BK;

// 32 K bytes (logical 16-byte chunks c0, c0+1) of staged row `row` under the
// SW = 2 swizzle of stage_group (key (row % 8) ^ ((row / 8) % 2); the slab
// offsets of the wave tiles are multiples of 64 rows, which keep it).
__device__ __forceinline__ v8i frag(const uint8_t* slab, int row, int c0) {
  const int sw = (row & 7) ^ ((row >> 3) & 1);
  const v4i lo = *reinterpret_cast<const v4i*>(slab + row * BK + ((c0 ^ sw) << 4));
  const v4i hi = *reinterpret_cast<const v4i*>(slab + row * BK + (((c0 + 1) ^ sw) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// FMT bit 0: A is E5M2 (else E4M3), bit 1: B is E5M2; the instructions'
// operand-format fields (0 = E4M3, 1 = E5M2), no block-exponent scaling.
template <int FMT>
__device__ __forceinline__ v4f mfma16(const v8i& a, const v8i& b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, (v4f){}, FMT & 1, FMT >> 1, 0, 0, 0, 0);
}

template <int FMT>
__device__ __forceinline__ v16f mfma32(const v8i& a, const v8i& b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, (v16f){}, FMT & 1, FMT >> 1, 0, 0, 0, 0);
}

template <int G, int WTM, int WTN>
struct Acc;
template <int WTM, int WTN>
struct Acc<128, WTM, WTN> {
  v4f t[WTM / 16][WTN / 16];
};
template <int WTM, int WTN>
struct Acc<64, WTM, WTN> {
  v16f t[WTM / 32][WTN / 32];
};

// G is the K segment the matrix cores contract before each promotion (64 or
// 128). The scale blocks are sg x sg with sg = G << sshift: for g = 256 the
// G = 128 kernel promotes every 128 K with its 256-block's factor. ROWA: A's
// factors are per row, sa is [M][K/sg].
// LAYOUT bit 1: A stored [K,M]; bit 0: B stored [K,N] (M resp. N any
// length; B transposed on the 256- and 128-wide tiles). A transposed tile is
// staged as its 128 K rows and read with the transposing LDS read (frag_tr16
// / frag_tr in gemm_common.h); the K order inside a fragment is the NT order.
template <int G, int BN, int WM, int GROUP_M, int FMT, int EPI, bool ROWA, int LAYOUT>
__global__ __launch_bounds__(NT) void gemm_fp8_nt_big(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                      const float* __restrict__ sa, const float* __restrict__ sb,
                                                      uint16_t* __restrict__ out, int M, int N, int K, int tiles_m,
                                                      int tiles_n, int vec_store, int sshift,
                                                      const float* __restrict__ bias, int relu) {
  static_assert(G == 64 || G == 128, "granularity");
  constexpr int WN = NW / WM;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int STAGE = A_BYTES + BN * BK;
  constexpr int SEGS = BK / G;                    // K segments per step
  constexpr int SCL = ROWA ? NW * 256 : 0;        // per-row factors of a step: [SEGS][BM] FP32, one piece per wave
  constexpr int SLOT = STAGE + SCL;
  constexpr int LDC = BN + 8;  // bf16 pitch of an epilogue pass
  static_assert(WTM == 64 || WTM == 128, "a wave's rows lie in one 128-row scale block");
  // Every wave's columns lie in one 128- (or 256-) column scale block: the
  // tile width is a multiple of 128 and the wave width divides 128.
  static_assert(BN % 128 == 0 && WTN % 16 == 0 && 128 % WTN == 0, "a wave's columns lie in one scale block");
  static_assert(G == 128 || WTN == 64, "g = 64: one 64-column scale block per wave");
  static_assert(BN % 8 == 0 && BN / 8 <= 4 * NW, "B copies: at most four row groups per wave");
  static_assert(128 * LDC * 2 <= 2 * STAGE, "an epilogue pass must fit in the ring");
  static_assert(BM * SEGS <= NW * 64, "a step's row factors: one 64-entry piece per wave");
  static_assert((LAYOUT & 1) == 0 || BN == 256 || BN == 128, "transposed B: 256- or 128-byte K rows");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * SLOT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int grp = wave >> 2;  // copy-issue group: one wave per SIMD in each

  int ks, tmi, tni;
  map_tile<GROUP_M>(tiles_m, tiles_n, ks, tmi, tni);
  const int m0 = tmi * BM, n0 = tni * BN;

  const uint32_t uK = (uint32_t)K;
  const v4i ra = rsrc_words(a + (int64_t)m0 * K, (uint32_t)min(BM, M - m0) * uK);
  const v4i rb = rsrc_words(b + (int64_t)n0 * K, (uint32_t)min(BN, N - n0) * uK);

  const int nkb = K / G;  // K segments
  const int sg = G << sshift, nks = K / sg;  // scale blocks
  const int nsteps = (K + BK - 1) / BK;
  const v4i rsa = ROWA ? rsrc_words(sa + (int64_t)m0 * nks, (uint32_t)min(BM, M - m0) * (uint32_t)nks * 4u) : (v4i){};

  // Scale rows of this wave. Blocks past the edge clamp to the last block
  // (their data is zero). g >= 128: one A block and one B block. g = 64: A
  // blocks of rows wr0 and wr0 + 64, one B block.
  const int wr0 = m0 + wm * WTM, wc0 = n0 + wn * WTN;
  const int lastm = (M - 1) / sg, lastn = (N - 1) / sg;
  const float* const sa0 = sa + (int64_t)min(wr0 / sg, lastm) * nks;
  const float* const sa1 = sa + (int64_t)min((wr0 + 64) / sg, lastm) * nks;
  const int bn0 = wc0 / sg;
  const float* const sb0 = sb + (int64_t)min(bn0, lastn) * nks;

  Acc<G, WTM, WTN> acc;
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

  // This wave's share of a step's copies: A row groups 8i + wave (i < 4) and
  // B row groups 8i + wave below BN / 8, into the slot of step t.
  auto issue_step = [&](int t) {
    uint8_t* slot = smem + (t & 1) * SLOT;
    if (ROWA && wave * 64 < BM * SEGS)  // pieces past the factors would only write padding
      stage_row_scales<BM, SEGS>(rsa, slot + STAGE, (uint32_t)nks, (uint32_t)((t * SEGS) >> sshift), wave, lane);
    const int64_t k0 = (int64_t)t * BK;
    if constexpr ((LAYOUT & 2) != 0) {
      // the step's K rows of A^T from column m0; past the tensor reads zero
      const v4i rat = rsrc_words(a + k0 * M + m0, tile_range_t(k0, K, M, m0, BK));
#pragma unroll
      for (int i = 0; i < 4; ++i) stage_group_t<BM>(rat, slot, (uint32_t)M, i * NW + wave, lane);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) stage_group<2>(ra, slot, uK, (uint32_t)t * BK, i * NW + wave, lane);
    }
    if constexpr ((LAYOUT & 1) != 0) {
      const v4i rbt = rsrc_words(b + k0 * N + n0, tile_range_t(k0, K, N, n0, BK));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i * NW + wave < BN / 8) stage_group_t<BN>(rbt, slot + A_BYTES, (uint32_t)N, i * NW + wave, lane);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i * NW + wave < BN / 8) stage_group<2>(rb, slot + A_BYTES, uK, (uint32_t)t * BK, i * NW + wave, lane);
    }
  };

  // The epilogue's bias for this lane's columns, loaded before the first
  // copies: the step waits cover it, and no output store is in flight when
  // the epilogue reads it. The plain form (EPI 0) loads and holds nothing.
  constexpr int NBJ = G == 128 ? WTN / 16 : WTN / 32;
  const bool hb = EPI != 0 && bias != nullptr;
  float bj[NBJ];
#pragma unroll
  for (int j = 0; j < NBJ; ++j) {
    const int col = wc0 + (G == 128 ? j * 16 + (lane & 15) : j * 32 + (lane & 31));
    bj[j] = hb && col < N ? bias[col] : 0.0f;
  }

  issue_step(0);

  for (int s = 0; s < nsteps; ++s) {
    DG_WAIT_VMCNT(0);  // this wave's part of step s has landed
    __syncthreads();   // all of step s visible; the other slot is free
    if constexpr (LAYOUT != 0) {
      // the tensor's last K row of a transposed operand whose stored row
      // length is not a multiple of 4 (see patch_tail_t)
      if (s == nsteps - 1 && (((LAYOUT & 2) && (M & 3)) || ((LAYOUT & 1) && (N & 3)))) {
        if (wave == 0) {
          uint8_t* slot = smem + (s & 1) * SLOT;
          const int64_t k0 = (int64_t)s * BK;
          if ((LAYOUT & 2) && (M & 3)) patch_tail_t<BM>(slot, a, (int64_t)K * M, M, k0, m0, lane);
          if ((LAYOUT & 1) && (N & 3)) patch_tail_t<BN>(slot + A_BYTES, b, (int64_t)K * N, N, k0, n0, lane);
        }
        __syncthreads();
      }
    }
    auto issue_next = [&](int who) {
      if (s + 1 < nsteps && grp == who) issue_step(s + 1);
    };
    const uint8_t* As = smem + (s & 1) * SLOT + wm * WTM * BK;
    const uint8_t* Bs = smem + (s & 1) * SLOT + A_BYTES + wn * WTN * BK;
    const uint8_t* At = smem + (s & 1) * SLOT;            // transposed tiles: K rows of the whole tile
    const uint8_t* Bt = smem + (s & 1) * SLOT + A_BYTES;
    // this lane's 16x16x128 fragment of A row block i / B column block j
    auto fa16 = [&](int i, int r16, int q) {
      if constexpr ((LAYOUT & 2) != 0) return frag_tr16<BM>(At, wm * WTM + i * 16, 0, lane);
      else return frag(As, i * 16 + r16, 2 * q);
    };
    auto fb16 = [&](int j, int r16, int q) {
      if constexpr ((LAYOUT & 1) != 0) return frag_tr16<BN>(Bt, wn * WTN + j * 16, 0, lane);
      else return frag(Bs, j * 16 + r16, 2 * q);
    };
    // ... and 32x32x64 fragment of the 64-byte K chunk h
    auto fa32 = [&](int i, int r32, int h, int h2) {
      if constexpr ((LAYOUT & 2) != 0) return frag_tr<BM>(At, wm * WTM + i * 32, 64 * h, lane);
      else return frag(As, i * 32 + r32, 4 * h + 2 * h2);
    };
    auto fb32 = [&](int j, int r32, int h, int h2) {
      if constexpr ((LAYOUT & 1) != 0) return frag_tr<BN>(Bt, wn * WTN + j * 32, 64 * h, lane);
      else return frag(Bs, j * 32 + r32, 4 * h + 2 * h2);
    };
    const float* scl = reinterpret_cast<const float*>(smem + (s & 1) * SLOT + STAGE);  // [SEGS][BM] (ROWA)

    if constexpr (G == 128) {
      // Slots t = (row block i, column block j). Slot t issues MFMA t and the
      // promotion of slot t - LAG, whose result has had LAG MFMAs' time to
      // land. Left alone, the scheduler puts each FMA right behind its own
      // MFMA and waits out the MFMA latency. LAG 7 measured about 0.5% faster
      // than 2, 3 or 5 on 8192^3 (the result ring costs 32 registers, no spill).
      constexpr int LAG = 7;
      constexpr int NJ = WTN / 16, SLOTS = (WTM / 16) * NJ, DSLOT = SLOTS / 4;
      const int r16 = lane & 15, q = lane >> 4;
      const int ksc = s >> sshift;
      const float a_s = ROWA ? 0.0f : sa0[ksc];
      const float sbv0 = sb0[ksc];
      const float sc0 = a_s * sbv0;
      // ROWA: factors of rows 16i + 4q .. +3 of the wave tile, read one row block ahead
      const float* const srow = scl + wm * WTM + 4 * q;
      v4f sr[WTM / 16], fr;
      if constexpr (ROWA) sr[0] = *reinterpret_cast<const v4f*>(srow);
      v8i bf[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = fb16(j, r16, q);
      v8i a_cur = fa16(0, r16, q), a_nxt = a_cur;
      v4f pr[LAG + 1];
#pragma unroll
      for (int t = 0; t < SLOTS + LAG; ++t) {
        const int i = t / NJ, j = t % NJ;
        if (t == 0) issue_next(0);
        if (t == DSLOT) issue_next(1);
        if (t < SLOTS) {
          if (j == 0 && i + 1 < WTM / 16) {
            a_nxt = fa16(i + 1, r16, q);
            if constexpr (ROWA) sr[i + 1] = *reinterpret_cast<const v4f*>(srow + (i + 1) * 16);
          }
          pr[t % (LAG + 1)] = mfma16<FMT>(a_cur, bf[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (t >= LAG) {
          const int u = t - LAG, ui = u / NJ, uj = u % NJ;
          if constexpr (ROWA) {
            // the row block's products, shared by its column blocks
            if (uj == 0) fr = sr[ui] * sbv0;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc.t[ui][uj][v] = __builtin_fmaf(pr[u % (LAG + 1)][v], fr[v], acc.t[ui][uj][v]);
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc.t[ui][uj][v] = __builtin_fmaf(pr[u % (LAG + 1)][v], sc0, acc.t[ui][uj][v]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (t < SLOTS && j == NJ - 1) a_cur = a_nxt;
      }
    } else {
      // The same schedule over the 32 x 32 blocks of each segment; waves 4-7
      // issue their copies at the second segment. With per-row factors on the
      // 256-wide tile (16 more registers per row block in flight) the
      // promotion runs one MFMA behind instead of two, which keeps the kernel
      // inside 256 registers.
      // 64-row wave tiles (256x128 tiles) have the registers for a lag of 3,
      // measured about 1.3% faster than 2 on 2000x4000x16384 (4: no better).
      constexpr int LAG = ROWA && BN == 256 ? 1 : (WTM == 64 ? 3 : 2);
      constexpr int NJ = WTN / 32, SLOTS = (WTM / 32) * NJ;
      const int r32 = lane & 31, h2 = lane >> 5;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = 2 * s + h;
        issue_next(h);
        if (kb < nkb) {  // K % 128 == 64: the last step holds one segment
          const float sbv = sb0[kb];
          const float f0 = ROWA ? 0.0f : sa0[kb] * sbv, f1 = ROWA ? 0.0f : sa1[kb] * sbv;
          // ROWA: factors of rows 32i + 8(v/4) + 4*h2 + v%4, read with the row
          // block's first MFMA
          const float* const srow = scl + h * BM + wm * WTM + 4 * h2;
          v4f sr[WTM / 32][4];
          float fr[16];
          v8i bf[NJ];
#pragma unroll
          for (int j = 0; j < NJ; ++j) bf[j] = fb32(j, r32, h, h2);
          v8i a_cur = fa32(0, r32, h, h2), a_nxt = a_cur;
          v16f pr[LAG + 1];
#pragma unroll
          for (int t = 0; t < SLOTS + LAG; ++t) {
            const int i = t / NJ, j = t % NJ;
            if (t < SLOTS) {
              if (j == 0 && i + 1 < WTM / 32) a_nxt = fa32(i + 1, r32, h, h2);
              if (ROWA && j == 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c) sr[i][c] = *reinterpret_cast<const v4f*>(srow + i * 32 + 8 * c);
              }
              pr[t % (LAG + 1)] = mfma32<FMT>(a_cur, bf[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (t >= LAG) {
              const int u = t - LAG, ui = u / NJ, uj = u % NJ;
              if constexpr (ROWA) {
                if (uj == 0) {  // the row block's products, shared by its column blocks (one B block per wave)
#pragma unroll
                  for (int v = 0; v < 16; ++v) fr[v] = sr[ui][v >> 2][v & 3] * sbv;
                }
#pragma unroll
                for (int v = 0; v < 16; ++v)
                  acc.t[ui][uj][v] = __builtin_fmaf(pr[u % (LAG + 1)][v], fr[v], acc.t[ui][uj][v]);
              } else {
                const float f = ui < 2 ? f0 : f1;  // rows 64.. of a 128-row wave tile use the next A block
#pragma unroll
                for (int v = 0; v < 16; ++v)
                  acc.t[ui][uj][v] = __builtin_fmaf(pr[u % (LAG + 1)][v], f, acc.t[ui][uj][v]);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (t < SLOTS && j == NJ - 1) a_cur = a_nxt;
          }
        }
      }
    }
    DG_STEP_SYNC_WG();
  }
  DG_WAIT_VMCNT(0);
  // Bias and activation in place, by all eight waves at once (the passes
  // below keep half of them idle).
  if constexpr (EPI != 0) {
    if constexpr (G == 128) {
#pragma unroll
      for (int j = 0; j < WTN / 16; ++j)
#pragma unroll
        for (int i = 0; i < WTM / 16; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc.t[i][j][v] = epilogue_fn<EPI>(acc.t[i][j][v], hb, bj[j], relu);
    } else {
#pragma unroll
      for (int j = 0; j < WTN / 32; ++j)
#pragma unroll
        for (int i = 0; i < WTM / 32; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc.t[i][j][v] = epilogue_fn<EPI>(acc.t[i][j][v], hb, bj[j], relu);
    }
  }

  // Epilogue, two passes of 128 rows: the waves whose rows lie in the pass
  // write their BF16 sub-tiles to LDS, then all threads store the pass.
  uint16_t* cs = reinterpret_cast<uint16_t*>(smem);
  const int prow = wm * WTM % 128;  // first row of this wave inside its pass

#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    if (wm * WTM / 128 == pass) {
      if constexpr (G == 128) {
        const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
        for (int j = 0; j < WTN / 16; ++j)
#pragma unroll
          for (int i = 0; i < WTM / 16; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              cs[(prow + i * 16 + 4 * q + v) * LDC + wn * WTN + j * 16 + r16] =
                  bf16_bits(acc.t[i][j][v]);
      } else {
        const int r32 = lane & 31, h2 = lane >> 5;
#pragma unroll
        for (int j = 0; j < WTN / 32; ++j)
#pragma unroll
          for (int i = 0; i < WTM / 32; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              cs[(prow + i * 32 + 8 * (v >> 2) + 4 * h2 + (v & 3)) * LDC + wn * WTN + j * 32 + r32] =
                  bf16_bits(acc.t[i][j][v]);
      }
    }
    __syncthreads();
    constexpr int CHUNKS = 128 * BN / 8;
    static_assert(CHUNKS % NT == 0, "epilogue chunks split evenly over the threads");
#pragma unroll
    for (int it = 0; it < CHUNKS / NT; ++it) {
      const int idx = it * NT + threadIdx.x;
      const int r = idx / (BN / 8), c = (idx % (BN / 8)) * 8;
      const int gr = m0 + pass * 128 + r, gc = n0 + c;
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

template <int G, int BN, int WM, int FMT, int EPI, bool ROWA, int LAYOUT>
hipError_t launch_fa(const GemmArgs& p, hipStream_t stream) {
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_fp8_nt_big<G, BN, WM, 4, FMT, EPI, ROWA, LAYOUT>), dim3(tiles_m * tiles_n), dim3(NT), 0, stream, p.a,
                     p.b, p.sa, p.sb, p.out, (int)p.M, (int)p.N, (int)p.K, tiles_m, tiles_n, p.vec_store, p.sshift,
                     p.bias, p.act == 1 ? 1 : 0);
  return hipGetLastError();
}

// RS selects the A factor forms compiled: 0 both, chosen by p.rowa (the NT
// entries); 1 g x g blocks only; 2 per-row factors only (the transposed
// layouts compile the two forms in separate translation units).
template <int G, int BN, int WM, int FMT, int EPI, int LAYOUT, int RS>
hipError_t launch_sa(const GemmArgs& p, hipStream_t stream) {
  if constexpr (RS == 1) {
    return p.rowa ? hipErrorInvalidValue : launch_fa<G, BN, WM, FMT, EPI, false, LAYOUT>(p, stream);
  } else if constexpr (RS == 2) {
    return p.rowa ? launch_fa<G, BN, WM, FMT, EPI, true, LAYOUT>(p, stream) : hipErrorInvalidValue;
  } else {
    return p.rowa ? launch_fa<G, BN, WM, FMT, EPI, true, LAYOUT>(p, stream)
                  : launch_fa<G, BN, WM, FMT, EPI, false, LAYOUT>(p, stream);
  }
}

template <int G, int BN, int WM, int FMT, int LAYOUT, int RS>
hipError_t launch_fmt(const GemmArgs& p, hipStream_t stream) {
  switch (epilogue_form(p.bias, p.act)) {
    case 0: return launch_sa<G, BN, WM, FMT, 0, LAYOUT, RS>(p, stream);
    case 1: return launch_sa<G, BN, WM, FMT, 1, LAYOUT, RS>(p, stream);
    case 2: return launch_sa<G, BN, WM, FMT, 2, LAYOUT, RS>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int G, int BN, int WM, int LAYOUT, int RS>
hipError_t launch_l(const GemmArgs& p, hipStream_t stream) {
  if (p.ksplit != 1 || p.sshift < 0 || p.sshift > 1) return hipErrorInvalidValue;
  switch (p.fmt) {
    case 0: return launch_fmt<G, BN, WM, 0, LAYOUT, RS>(p, stream);
    case 1: return launch_fmt<G, BN, WM, 1, LAYOUT, RS>(p, stream);
    case 2: return launch_fmt<G, BN, WM, 2, LAYOUT, RS>(p, stream);
    case 3: return launch_fmt<G, BN, WM, 3, LAYOUT, RS>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// The NT table entries.
template <int G, int BN, int WM>
hipError_t launch(const GemmArgs& p, hipStream_t stream) {
  return p.layout == 0 ? launch_l<G, BN, WM, 0, 0>(p, stream) : hipErrorInvalidValue;
}

// The transposed layouts on the same tile, with the A factor form RS
// (instantiated in gemm_fp8_big_layouts.hip and gemm_fp8_big_layouts_rowa.hip).
template <int G, int BN, int WM, int RS>
hipError_t launch_layout(const GemmArgs& p, hipStream_t stream) {
  switch (p.layout) {
    case 1: return launch_l<G, BN, WM, 1, RS>(p, stream);
    case 2: return launch_l<G, BN, WM, 2, RS>(p, stream);
    case 3: return launch_l<G, BN, WM, 3, RS>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace big

}  // namespace dg
