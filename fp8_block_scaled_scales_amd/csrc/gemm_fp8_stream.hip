// Small-M block-scaled FP8 GEMM for gfx950 that streams B once, without a
// reduction across workgroups.
//
// Same operation as the other kernels (DeepGEMM实战 §2.2: FP32 scale per g x g
// block, restored during accumulation; §3.2: FP32 accumulation per K segment,
// the segments then added; §3.3/§4.2: NT layout, A [M,K], B [N,K], BF16 out).
//
// With M this small the GEMM is a stream of B from HBM, and the way to reach
// HBM speed is to spread B over every CU with many bytes in flight
// (DeepGEMM实战 §5.3 names too little parallelism as the problem of small
// shapes). One workgroup owns a 32 x 32 output tile over the whole K (M = 64,
// N = 4096 gives 256 workgroups). Its four waves split the K steps (wave w
// takes steps w, w+4, ...), each with a private ring of four LDS slots fed by
// HBM->LDS copies: a wave waits only for its own copies, so the main loop has
// no barrier (A, which stays in L2, and B, which streams from HBM, have
// rings of different depths). Each wave accumulates the whole 32 x 32 tile over its steps
// (one 32x32x64 MFMA per 64-wide K segment, promoted by sa*sb into an FP32
// accumulator); at the end the four partial tiles are added through LDS in
// wave order, so results do not depend on timing, and written as BF16.
//
// Per CU this reads 32 rows of A and 32 rows of B over the whole K (458 KB for
// K = 7168); A comes from L2 after its first touch, so HBM sees B once.
//
// Per-row A factors (ROWA; one factor per row of A and K segment, the
// template article's per-channel choice, §3.4): each A slot carries the
// step's 32 (g >= 128) or 64 (g = 64) row factors, copied ahead of the slab
// by one 4-byte-per-lane copy; the B ring gives up a slot to make room.
//
// Transposed operands (LAYOUT; DeepGEMM实战 §3.3: A stored [K,M] and/or B
// stored [K,N]): a step's tile of such an operand is its 128 K rows of 32
// bytes, copied with the same number of 16-byte-per-lane copies as the NT
// slab (32 K rows per copy) and read with the transposing LDS read. Eight
// such rows are 256 contiguous bytes, all banks once, so these slabs need no
// swizzle. The fragments hold the same K bytes in the same order as the NT
// ones, so every layout gives the NT bits.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "gemm_fp8_nt.h"

namespace dg {

namespace stream {

constexpr int BM = 32, BN = 32, BK = 128;
constexpr int NW = 4;
constexpr int A_SLAB = BM * BK, B_SLAB = BN * BK;  // 4 KB each per step

// Per wave: A slabs (L2 hits after their first touch) are copied two steps
// ahead into a 3-slot ring, B slabs (streamed from HBM, whose loaded latency
// is several microseconds) six steps ahead into a 7-slot ring. 40 KB per
// wave, the whole 160 KB LDS for four waves. With per-row A factors each A
// slot also holds the step's factors (256 bytes) and B keeps 6 slots.
template <bool ROWA>
struct Ring {
  static constexpr int A_SLOTS = 3, B_SLOTS = ROWA ? 6 : 7;
  static constexpr int A_AHEAD = A_SLOTS - 1, B_AHEAD = B_SLOTS - 1;
  static constexpr int SA_SLAB = ROWA ? 256 : 0;            // [SEGS][32] FP32 row factors of the step
  static constexpr int A_PITCH = A_SLAB + SA_SLAB;          // one A slot
  static constexpr int WAVE_LDS = A_SLOTS * A_PITCH + B_SLOTS * B_SLAB;
  // copy instructions per step and operand (one wave); the factor copy goes with A, ahead of it
  static constexpr int A_LOADS = BM / 8 + (ROWA ? 1 : 0), B_LOADS = BN / 8;
  // Issue order per iteration t: A(t + A_AHEAD), then B(t + B_AHEAD). Waiting
  // for A(t) (the later-issued of A(t), B(t)) leaves in flight what followed
  // it: B(t + B_AHEAD - A_AHEAD), then the copies of A_AHEAD - 1 more
  // iterations.
  static constexpr int WAIT_AFTER_A = (A_AHEAD - 1) * (A_LOADS + B_LOADS) + B_LOADS;
  static_assert(NW * WAVE_LDS <= 160 * 1024, "LDS");
  static_assert(A_AHEAD * (A_LOADS + B_LOADS) + (B_AHEAD - A_AHEAD) * B_LOADS < 64, "vmcnt range");
};

// Descriptor over step st's tile of an operand stored [K, len], from column
// col0 (see tile_range_t); steps past the end get an empty range, so their
// copies move nothing.
__device__ __forceinline__ v4i step_rsrc_t(const uint8_t* base, int K, int len, int col0, int st, int nsteps) {
  const int64_t k0 = (int64_t)st * BK;
  return st < nsteps ? rsrc_words(base + k0 * len + col0, tile_range_t(k0, K, len, col0, BK)) : rsrc_words(base, 0);
}

__device__ __forceinline__ v8i frag(const uint8_t* slab, int row, int c0) {
  const int sw = (row >> 1) & 7;
  const v4i lo = *reinterpret_cast<const v4i*>(slab + row * BK + ((c0 ^ sw) << 4));
  const v4i hi = *reinterpret_cast<const v4i*>(slab + row * BK + (((c0 + 1) ^ sw) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// G: K segment contracted before each promotion; scale blocks sg = G << sshift
// (g = 256 runs the G = 128 kernel with one factor per two segments). FMT bit
// 0: A is E5M2 (else E4M3), bit 1: B is E5M2. ROWA: A's factors are per row,
// sa is [M][K/sg]. LAYOUT bit 1: A stored [K,M]; bit 0: B stored [K,N].
template <int G, int FMT, int EPI, bool ROWA, int LAYOUT>
__global__ __launch_bounds__(64 * NW) void gemm_fp8_stream(const uint8_t* __restrict__ a,
                                                              const uint8_t* __restrict__ b,
                                                              const float* __restrict__ sa,
                                                              const float* __restrict__ sb,
                                                              uint16_t* __restrict__ out, int M, int N, int K,
                                                              int tiles_m, int tiles_n, int sshift,
                                                              const float* __restrict__ bias, int relu) {
  static_assert(G == 64 || G == 128, "granularity");
  constexpr bool TA = (LAYOUT & 2) != 0, TB = (LAYOUT & 1) != 0;
  using R = Ring<ROWA>;
  constexpr int SEGS = BK / G;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NW * R::WAVE_LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int ks, tmi, tni;
  map_tile<2>(tiles_m, tiles_n, ks, tmi, tni);
  const int m0 = tmi * BM, n0 = tni * BN;
  const uint32_t uK = (uint32_t)K;
  // NT operands: one descriptor over the tile's rows for the whole K
  // (transposed ones take one per step, step_rsrc_t)
  const v4i ra = TA ? (v4i){} : rsrc_words(a + (int64_t)m0 * K, (uint32_t)min(BM, M - m0) * uK);
  const v4i rb = TB ? (v4i){} : rsrc_words(b + (int64_t)n0 * K, (uint32_t)min(BN, N - n0) * uK);

  const int nkb = K / G;
  const int sg = G << sshift, nks = K / sg;
  const int nsteps = (K + BK - 1) / BK;
  // 32 rows starting at a multiple of 32 lie in one g-block (g >= 64).
  const float* const sa_row = sa + (int64_t)(m0 / sg) * nks;
  const float* const sb_row = sb + (int64_t)(n0 / sg) * nks;
  const v4i rsa = ROWA ? rsrc_words(sa + (int64_t)m0 * nks, (uint32_t)min(BM, M - m0) * (uint32_t)nks * 4u) : (v4i){};

  // The epilogue's bias for this lane's column, loaded first: it is older
  // than every copy below, so the copies' waits cover it, and no output store
  // is in flight when the epilogue reads it.
  const int ocol = n0 + (lane & 31);
  const bool hb = EPI != 0 && bias != nullptr;
  const float bc = hb && ocol < N ? bias[ocol] : 0.0f;

  uint8_t* const a_ring = smem + wave * R::WAVE_LDS;
  uint8_t* const b_ring = a_ring + R::A_SLOTS * R::A_PITCH;
  // This wave's step t is global step wave + NW*t. Steps past the end issue
  // copies of nothing, so every wait below counts exactly.
  auto issue_a = [&](int t) {
    const int st = wave + NW * t;
    uint8_t* const slot = a_ring + (t % R::A_SLOTS) * R::A_PITCH;
    if constexpr (ROWA)
      stage_row_scales<BM, SEGS>(rsa, slot + A_SLAB, (uint32_t)nks, (uint32_t)((st * SEGS) >> sshift), 0, lane,
                                 st < nsteps);
    if constexpr (TA) {
      const v4i rat = step_rsrc_t(a, K, M, m0, st, nsteps);
#pragma unroll
      for (int g = 0; g < BK / 32; ++g) stage_group_t<BM>(rat, slot, (uint32_t)M, g, lane);
    } else {
#pragma unroll
      for (int g = 0; g < BM / 8; ++g) stage_group<1>(ra, slot, uK, (uint32_t)st * BK, g, lane, st < nsteps);
    }
  };
  auto issue_b = [&](int t) {
    const int st = wave + NW * t;
    uint8_t* const slot = b_ring + (t % R::B_SLOTS) * B_SLAB;
    if constexpr (TB) {
      const v4i rbt = step_rsrc_t(b, K, N, n0, st, nsteps);
#pragma unroll
      for (int g = 0; g < BK / 32; ++g) stage_group_t<BN>(rbt, slot, (uint32_t)N, g, lane);
    } else {
#pragma unroll
      for (int g = 0; g < BN / 8; ++g) stage_group<1>(rb, slot, uK, (uint32_t)st * BK, g, lane, st < nsteps);
    }
  };
  // The lane's 32x32x64 fragment of K half q (K bytes 64q + 32*(lane/32) ..
  // +31 of the step) from a slab, NT or transposed.
  auto frag_a = [&](const uint8_t* s, int q) {
    if constexpr (TA) return frag_tr<BM>(s, 0, 64 * q, lane);
    else return frag(s, lane & 31, 4 * q + 2 * (lane >> 5));
  };
  auto frag_b = [&](const uint8_t* s, int q) {
    if constexpr (TB) return frag_tr<BN>(s, 0, 64 * q, lane);
    else return frag(s, lane & 31, 4 * q + 2 * (lane >> 5));
  };

  v16f acc = {};
  // acc += p * (A factor * B factor): one block product, or (ROWA) the lane's
  // sixteen row factors from LDS, each times the B factor.
  auto promote = [&](const v16f& p, const float* fr, float sbv, float sav) {
    if constexpr (ROWA) {
      v4f r[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) r[c] = *reinterpret_cast<const v4f*>(fr + 8 * c);
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = __builtin_fmaf(p[v], r[v >> 2][v & 3] * sbv, acc[v]);
    } else {
      const float sc = sav * sbv;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = __builtin_fmaf(p[v], sc, acc[v]);
    }
  };
  const int my_steps = nsteps > wave ? (nsteps - wave + NW - 1) / NW : 0;
  // Prologue in the steady-state order: B(0) .. B(B_AHEAD - A_AHEAD - 1), then
  // for j = 0 .. A_AHEAD-1 the pair A(j), B(B_AHEAD - A_AHEAD + j).
#pragma unroll
  for (int t = 0; t < R::B_AHEAD - R::A_AHEAD; ++t) issue_b(t);
#pragma unroll
  for (int j = 0; j < R::A_AHEAD; ++j) {
    issue_a(j);
    issue_b(R::B_AHEAD - R::A_AHEAD + j);
  }

  // g = 64: the factors of this wave's next step, read a step ahead. Scalar
  // loads share the counter the fragment reads wait on, so a load issued
  // where its value is needed stalls the wave for its whole latency, and at
  // g = 64 that happened twice per step (3-15% of the time on streaming
  // shapes). At g = 128, one load per step, reading ahead measured 2-4%
  // slower and the factors are read in place. The read after the last step
  // clamps to the last segment.
  float nsa[SEGS], nsb[SEGS];
  auto load_factors = [&](int t) {
    const int st = wave + NW * t;
#pragma unroll
    for (int h = 0; h < SEGS; ++h) {
      const int kb = min(2 * st + h, nkb - 1);
      nsa[h] = sa_row[kb];
      nsb[h] = sb_row[kb];
    }
  };
  if (G == 64 && my_steps > 0) load_factors(0);

  const int h2 = lane >> 5;
  for (int t = 0; t < my_steps; ++t) {
    DG_WAIT_VMCNT(R::WAIT_AFTER_A);  // A(t) and the earlier-issued B(t) have landed
    const int st = wave + NW * t;
    float csa[SEGS], csb[SEGS];
    if constexpr (G == 64) {
#pragma unroll
      for (int h = 0; h < SEGS; ++h) {
        csa[h] = nsa[h];
        csb[h] = nsb[h];
      }
      load_factors(t + 1);
    }
    uint8_t* const As = a_ring + (t % R::A_SLOTS) * R::A_PITCH;
    uint8_t* const Bs = b_ring + (t % R::B_SLOTS) * B_SLAB;
    if constexpr (LAYOUT != 0) {
      // the tensor's last K row of a transposed operand whose stored row
      // length is not a multiple of 4 (see patch_tail_t); the slots are this
      // wave's own, so its own copies having landed is enough
      if (st == nsteps - 1) {
        const int64_t k0 = (int64_t)st * BK;
        if (TA && (M & 3)) patch_tail_t<BM>(As, a, (int64_t)K * M, M, k0, m0, lane);
        if (TB && (N & 3)) patch_tail_t<BN>(Bs, b, (int64_t)K * N, N, k0, n0, lane);
      }
    }
    // ROWA: factors [SEGS][32] of the step; this lane's rows 8c + 4*h2 .. +3
    const float* const srow = reinterpret_cast<const float*>(As + A_SLAB) + 4 * h2;
#pragma unroll
    for (int h = 0; h < BK / 64; ++h) {
      const int kb = G == 128 ? st : 2 * st + h;
      if (G == 64 && kb >= nkb) break;  // K % 128 == 64: the last step holds one segment
      const v8i af = frag_a(As, h);
      const v8i bf = frag_b(Bs, h);
      if (G == 128) {
        if (h == 0) {
          // the segment is the whole step: chain both halves, then promote once
          const v8i af1 = frag_a(As, 1);
          const v8i bf1 = frag_b(Bs, 1);
          v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, (v16f){}, FMT & 1, FMT >> 1, 0, 0, 0, 0);
          p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af1, bf1, p, FMT & 1, FMT >> 1, 0, 0, 0, 0);
          promote(p, srow, sb_row[kb >> sshift], sa_row[kb >> sshift]);
        }
      } else {
        const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, (v16f){}, FMT & 1, FMT >> 1, 0, 0, 0, 0);
        promote(p, srow + 32 * h, csb[h], csa[h]);
      }
    }
    DG_STEP_SYNC_WAVE();
    // Refill the slots of step t-1, read by this wave only and done with one
    // iteration ago.
    issue_a(t + R::A_AHEAD);
    issue_b(t + R::B_AHEAD);
  }
  DG_WAIT_VMCNT(0);  // copies of nothing issued past this wave's last step

  // Add the four waves' partial tiles in wave order, through LDS.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [NW][16][64]
#pragma unroll
  for (int v = 0; v < 16; ++v) red[(wave * 16 + v) * 64 + lane] = acc[v];
  __syncthreads();
  if (wave != 0) return;
  uint16_t res[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float tsum = red[v * 64 + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) tsum += red[(w * 16 + v) * 64 + lane];
    res[v] = bf16_bits(epilogue_fn<EPI>(tsum, hb, bc, relu));
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = m0 + 8 * (v >> 2) + 4 * h2 + (v & 3);
    if (row < M && ocol < N) out[(int64_t)row * N + ocol] = res[v];
  }
}

template <int G, int FMT, int EPI, bool ROWA, int LAYOUT>
hipError_t launch_fa(const GemmArgs& p, hipStream_t stream) {
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_fp8_stream<G, FMT, EPI, ROWA, LAYOUT>), dim3(tiles_m * tiles_n), dim3(64 * NW), 0, stream,
                     p.a, p.b, p.sa, p.sb, p.out, (int)p.M, (int)p.N, (int)p.K, tiles_m, tiles_n, p.sshift, p.bias,
                     p.act == 1 ? 1 : 0);
  return hipGetLastError();
}

template <int G, int FMT, int EPI, int LAYOUT>
hipError_t launch_sa(const GemmArgs& p, hipStream_t stream) {
  return p.rowa ? launch_fa<G, FMT, EPI, true, LAYOUT>(p, stream) : launch_fa<G, FMT, EPI, false, LAYOUT>(p, stream);
}

template <int G, int FMT, int LAYOUT>
hipError_t launch_fmt(const GemmArgs& p, hipStream_t stream) {
  switch (epilogue_form(p.bias, p.act)) {
    case 0: return launch_sa<G, FMT, 0, LAYOUT>(p, stream);
    case 1: return launch_sa<G, FMT, 1, LAYOUT>(p, stream);
    case 2: return launch_sa<G, FMT, 2, LAYOUT>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int G, int LAYOUT>
hipError_t launch_l(const GemmArgs& p, hipStream_t stream) {
  switch (p.fmt) {
    case 0: return launch_fmt<G, 0, LAYOUT>(p, stream);
    case 1: return launch_fmt<G, 1, LAYOUT>(p, stream);
    case 2: return launch_fmt<G, 2, LAYOUT>(p, stream);
    case 3: return launch_fmt<G, 3, LAYOUT>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
hipError_t launch(const GemmArgs& p, hipStream_t stream) {
  if (p.ksplit != 1 || p.sshift < 0 || p.sshift > 1) return hipErrorInvalidValue;
  switch (p.layout) {
    case 0: return launch_l<G, 0>(p, stream);
    case 1: return launch_l<G, 1>(p, stream);
    case 2: return launch_l<G, 2>(p, stream);
    case 3: return launch_l<G, 3>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace stream

// Every layout: the NT table entries (6, 7) and their transposed forms.
hipError_t launch_stream_g128(const GemmArgs& p, hipStream_t s) { return stream::launch<128>(p, s); }
hipError_t launch_stream_g64(const GemmArgs& p, hipStream_t s) { return stream::launch<64>(p, s); }

}  // namespace dg
