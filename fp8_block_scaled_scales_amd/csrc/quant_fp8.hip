// Block quantiser FP32, BF16 or FP16 -> FP8 (E4M3FN or E5M2) with one FP32
// scale per g x g block (or 1 x g segment), g = 64, 128 or 256, for gfx950.
// It produces the GEMM's inputs: the pages place quantisation outside the
// GEMM, say that activations must be quantised online and that the
// granularity must equal the GEMM's (DeepGEMM实战 §4.4), that one factor per
// block maps the block into FP8 range (§2.2) by dividing (§5.2), and name E4M3
// and E5M2 as the formats (§2.2).
//
// Per block: amax = max |x| over the elements present (edge blocks past the
// last row are partial), scale = amax / fmax (FP32, correctly rounded; 1.0
// where that is zero: an all-zero block, or amax so small the quotient
// underflows; fmax = 448 for E4M3, 57344 for E5M2), code =
// FP8(x / scale) with a correctly rounded FP32 divide and the hardware's
// round-to-nearest-even conversion, saturating at +-fmax (reached only where
// scale is subnormal and so coarsely rounded; otherwise |x / scale| <= fmax
// up to one rounding, which still rounds to fmax).
// The divide is taken as a reciprocal and two FMA corrections, which give the
// correctly rounded quotient (div_by_scale).
//
// 16-bit inputs (the weights and activations to quantise arrive in FP16 or
// BF16, DeepGEMM实战 §4.4) are widened exactly to FP32 as they are used; the
// rule is then the FP32 one, on the same values.
//
// One workgroup per block, 256 or 512 threads by block size (1024 for g =
// 256, and for a launch of at most 256 blocks). The block (64 KB of FP32 for g = 128) stays in
// registers, as loaded, between the amax pass and the encode pass, so x is
// read from HBM once: the kernel is bound by HBM bandwidth (4 or 2 bytes in,
// 1 byte out per element). Every load is 16 bytes: four FP32 or eight 16-bit
// elements per lane.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "quant_fp8.h"

namespace dg {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Input element kinds: 0 FP32, 1 BF16, 2 FP16 (the library's DG_IN_* codes).
template <int IN>
struct InKind {
  static constexpr int kBytes = IN == 0 ? 4 : 2;  // bytes per element
  static constexpr int kPerLoad = 16 / kBytes;     // elements per 16-byte load
  static constexpr int kQuads = kPerLoad / 4;      // groups of four per load
};

// Elements 4*H .. 4*H+3 of a 16-byte load, as FP32 (exact for every kind).
// A 32-bit word holds two 16-bit elements, the first in its low half. BF16 is
// the high half of an FP32 pattern; FP16 converts exactly.
template <int IN, int H>
__device__ __forceinline__ v4f widen(v4u w) {
  if constexpr (IN == 0) {
    return __builtin_bit_cast(v4f, w);
  } else {
    const unsigned a = H ? w.z : w.x, b = H ? w.w : w.y;
    if constexpr (IN == 1) {
      return (v4f){__uint_as_float(a << 16), __uint_as_float(a & 0xFFFF0000u), __uint_as_float(b << 16),
                   __uint_as_float(b & 0xFFFF0000u)};
    } else {
      const v2h ha = __builtin_bit_cast(v2h, a), hb = __builtin_bit_cast(v2h, b);
      return (v4f){(float)ha.x, (float)ha.y, (float)hb.x, (float)hb.y};
    }
  }
}

__device__ __forceinline__ float amax4(v4f v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v2u16 abs_bits2(unsigned w) { return __builtin_bit_cast(v2u16, w & 0x7FFF7FFFu); }

// max |x| over the elements of one 16-byte load. For 16-bit input the max is
// taken on the bit patterns: with the sign bit cleared, the patterns of
// finite BF16 or FP16 values order as the magnitudes do, so a packed 16-bit
// integer max finds the largest, which is then widened once. Nothing widened
// here stays live until the encode pass, which widens its own copies.
template <int IN>
__device__ __forceinline__ float amax_load(v4u w) {
  if constexpr (IN == 0) {
    return amax4(widen<IN, 0>(w));
  } else {
    const v2u16 m = __builtin_elementwise_max(__builtin_elementwise_max(abs_bits2(w.x), abs_bits2(w.y)),
                                              __builtin_elementwise_max(abs_bits2(w.z), abs_bits2(w.w)));
    const unsigned top = m.x > m.y ? m.x : m.y;
    if constexpr (IN == 1) return __uint_as_float(top << 16);
    else return (float)__builtin_bit_cast(_Float16, (unsigned short)top);
  }
}

// Division by a block's scale s, rounded as the correctly rounded FP32 divide
// rounds it, without a divide per element. inv = RN(1/s) is computed once per
// block (a correctly rounded divide); per element q0 = RN(x * inv) lies within
// 1.5 ulp of x/s, one correction q1 = RN(q0 + RN(x - q0*s) * inv) (the
// remainder exact under the FMA) brings it within one ulp, and a second
// correction then gives RN(x/s) by Markstein's theorem on FMA-based division
// (P. Markstein, "IA-64 and Elementary Functions", 2000; also the chapter on
// division with an FMA in the Handbook of Floating-Point Arithmetic): with a
// correctly rounded reciprocal and a quotient within one ulp, the corrected
// quotient is the correctly rounded one. The theorem asks that nothing
// overflows or underflows: s and 1/s normal (the caller's uniform test,
// recip_ok; blocks outside it divide per element) and x/s at most the
// format's largest value. A quotient in FP32's subnormal range may come out
// wrong in its last bits, but every such value is far below half the smallest
// FP8 subnormal and encodes to a signed zero either way; the sign is x's (an
// input -0 gives -0, where the corrections alone would give +0).
// A block's factor: amax / fmax (correctly rounded), or 1.0 where that is
// zero: an all-zero block, or one whose amax is so small that the quotient
// underflows (no factor of zero to divide by; 1.0 encodes its values, all
// below fmax * 2^-150, under 2^-134, as zeros).
__device__ __forceinline__ float block_scale(float amax, float fmax) {
  const float s = amax / fmax;
  return s > 0.0f ? s : 1.0f;
}

__device__ __forceinline__ bool recip_ok(float s) { return s >= 0x1p-120f && s <= 0x1p120f; }

__device__ __forceinline__ float div_by_scale(float x, float s, float inv) {
  float q = x * inv;
  q = __builtin_fmaf(__builtin_fmaf(-q, s, x), inv, q);
  q = __builtin_fmaf(__builtin_fmaf(-q, s, x), inv, q);
  return __builtin_copysignf(q, x);
}

// One DPP move of v across the wave (row_mask, bank_mask all on; every
// source lane exists for the patterns used here).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over each aligned group of L lanes (L = 8, 16, 32 or 64), in every lane
// of the group: within quads by two swaps (DPP quad_perm [1,0,3,2],
// [2,3,0,1]), then each lane against its mirror in the 8-lane half row, which
// leaves the half row's max in every lane, and in the 16-lane row (DPP
// row_half_mirror, row_mirror); beyond 16 lanes, cross-lane shuffles. max is
// exact and order-free.
template <int L>
__device__ __forceinline__ float group_max(float m) {
  static_assert(L == 8 || L == 16 || L == 32 || L == 64, "group");
  m = fmaxf(m, dpp_f<0xB1>(m));
  m = fmaxf(m, dpp_f<0x4E>(m));
  m = fmaxf(m, dpp_f<0x141>(m));
  if constexpr (L >= 16) m = fmaxf(m, dpp_f<0x140>(m));
  if constexpr (L >= 32) m = fmaxf(m, __shfl_xor(m, 16, 64));
  if constexpr (L >= 64) m = fmaxf(m, __shfl_xor(m, 32, 64));
  return m;
}

// Two FP8 codes of (x0, x1) packed into the low (HI = false) or high half of
// `old`: FMT 0 E4M3FN, 1 E5M2 (hardware round-to-nearest-even).
template <int FMT, bool HI>
__device__ __forceinline__ int cvt2(float x0, float x1, int old) {
  if constexpr (FMT == 1) return __builtin_amdgcn_cvt_pk_bf8_f32(x0, x1, old, HI);
  else return __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, old, HI);
}

// Four codes of v / s in one 32-bit word (bytes in element order). FAST (s
// and 1/s normal): |v / s| rounds to at most fmax, since s carries a relative
// error of at most 2^-24. Otherwise s is subnormal or tiny, its own rounding
// can be coarse enough that |v / s| passes fmax, and the quotient saturates
// to +-fmax as FP8's round-to-nearest with saturation takes it (the
// conversion instruction alone does not saturate).
template <int FMT, bool FAST>
__device__ __forceinline__ int encode4(v4f v, float s, float inv) {
  if constexpr (FAST) {
    const int lo = cvt2<FMT, false>(div_by_scale(v.x, s, inv), div_by_scale(v.y, s, inv), 0);
    return cvt2<FMT, true>(div_by_scale(v.z, s, inv), div_by_scale(v.w, s, inv), lo);
  } else {
    constexpr float FMAX = FMT == 1 ? 57344.0f : 448.0f;
    auto sat = [](float y) { return fminf(fmaxf(y, -FMAX), FMAX); };
    const int lo = cvt2<FMT, false>(sat(v.x / s), sat(v.y / s), 0);
    return cvt2<FMT, true>(sat(v.z / s), sat(v.w / s), lo);
  }
}

// The codes of one 16-byte load's elements, divided by s, stored at q (4 or
// 8 bytes: one code per element, in element order).
template <int FMT, int IN, bool FAST>
__device__ __forceinline__ void encode_store(v4u w, float s, float inv, uint8_t* q) {
  const int c0 = encode4<FMT, FAST>(widen<IN, 0>(w), s, inv);
  if constexpr (InKind<IN>::kQuads == 1) {
    *reinterpret_cast<int*>(q) = c0;
  } else {
    *reinterpret_cast<v2i*>(q) = (v2i){c0, encode4<FMT, FAST>(widen<IN, 1>(w), s, inv)};
  }
}

// NT threads per block: 256 or 512 by block size (launch_g), or up to 1024
// (no more than the block's 16-byte pieces) when the blocks are few enough
// that each CU holds at most one; g = 256 always takes 1024.
template <int G, int FMT, int IN, int NT>
__global__ __launch_bounds__(NT) void quant_fp8_blocks(const void* __restrict__ xv, uint8_t* __restrict__ q,
                                                       float* __restrict__ scales, int rows, int cols) {
  constexpr float FMAX = FMT == 1 ? 57344.0f : 448.0f;
  constexpr int EPL = InKind<IN>::kPerLoad;
  constexpr int ROW_L = G / EPL;              // lanes per block row
  constexpr int ROWS_PER_PASS = NT / ROW_L;   // block rows covered by one pass
  constexpr int PASSES = G / ROWS_PER_PASS;
  static_assert(PASSES * ROWS_PER_PASS == G, "passes");
  __shared__ float red[NT / 64];
  const char* x = static_cast<const char*>(xv);

  const int ncb = cols / G;
  const int rb = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  const int t = threadIdx.x;
  const int rsub = t / ROW_L, cl = t % ROW_L;
  const int col = cb * G + cl * EPL;

  v4u v[PASSES];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = rb * G + p * ROWS_PER_PASS + rsub;
    if (r < rows) {
      v[p] = *reinterpret_cast<const v4u*>(x + ((int64_t)r * cols + col) * InKind<IN>::kBytes);
    } else {
      v[p] = (v4u){0u, 0u, 0u, 0u};
    }
    amax = fmaxf(amax, amax_load<IN>(v[p]));
  }
  // max is exact and order-free: over the wave, then across the waves
  amax = group_max<64>(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) amax = fmaxf(amax, red[w]);
  const float scale = block_scale(amax, FMAX);
  if (t == 0) scales[blockIdx.x] = scale;

  const float inv = 1.0f / scale;
  const bool fast = recip_ok(scale);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = rb * G + p * ROWS_PER_PASS + rsub;
    if (r < rows) {
      uint8_t* dst = q + (int64_t)r * cols + col;
      if (fast) encode_store<FMT, IN, true>(v[p], scale, inv, dst);
      else encode_store<FMT, IN, false>(v[p], scale, inv, dst);
    }
  }
}

// 1 x g blocks (one factor per row and g-wide column segment; the per-row A
// factors of the template article's per-channel choice, §3.4): the same rule
// per segment. A lane loads 16 bytes (four FP32 or eight 16-bit elements), so
// g / 4 or g / 8 lanes own a segment and one load instruction of a wave
// covers 1 KB of consecutive input when a row has that much; amax is a
// butterfly over the segment's lanes. Each wave takes U such groups, all
// loads issued before any is used, so a thread has U x 16 bytes in flight.
// Segments are numbered row-major (row * cols/G + column block), which is
// also the factor's index in the [rows][cols/G] scale tensor; the host keeps
// their count below 2^31.
template <int G, int FMT, int IN, int U>
__global__ __launch_bounds__(256) void quant_fp8_rows(const void* __restrict__ xv, uint8_t* __restrict__ q,
                                                      float* __restrict__ scales, unsigned nseg, int cols) {
  constexpr float FMAX = FMT == 1 ? 57344.0f : 448.0f;
  constexpr int EPL = InKind<IN>::kPerLoad;
  constexpr int LPS = G / EPL;      // lanes per segment
  constexpr int SPW = 64 / LPS;     // segments per wave-wide load
  const char* x = static_cast<const char*>(xv);
  const int lane = threadIdx.x & 63;
  const int cl = lane % LPS;
  const unsigned ncb = (unsigned)(cols / G);
  // unsigned: the last workgroup's segments may pass 2^31 - 1 (and are not live)
  const unsigned wseg = (blockIdx.x * 4u + (threadIdx.x >> 6)) * (unsigned)(SPW * U);  // the wave's first segment
  const unsigned seg0 = wseg + (unsigned)(lane / LPS);
  // (row, column block) of the wave's first segment from one division; the
  // lane's segments follow it by at most SPW * U - 1, a few row wraps at most
  const unsigned wrow = wseg / ncb, wcb = wseg - wrow * ncb;
  v4u v[U];
  int64_t off[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const unsigned seg = seg0 + (unsigned)(u * SPW);
    unsigned row = wrow, cb = wcb + (seg - wseg);
    if (cb >= ncb) {
      const unsigned k = cb < 2 * ncb ? 1u : cb / ncb;
      row += k;
      cb -= k * ncb;
    }
    // whole segments are live or not, so each reduction stays inside live lanes
    off[u] = seg < nseg ? (int64_t)row * cols + cb * G + cl * EPL : 0;
    v[u] = seg < nseg ? *reinterpret_cast<const v4u*>(x + off[u] * InKind<IN>::kBytes) : (v4u){0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const unsigned seg = seg0 + (unsigned)(u * SPW);
    const float amax = group_max<LPS>(amax_load<IN>(v[u]));
    if (seg >= nseg) continue;
    const float scale = block_scale(amax, FMAX);
    if (cl == 0) scales[seg] = scale;
    // the segment's lanes agree on scale, so a divergent choice splits
    // whole segments
    if (recip_ok(scale)) encode_store<FMT, IN, true>(v[u], scale, 1.0f / scale, q + off[u]);
    else encode_store<FMT, IN, false>(v[u], scale, 0.0f, q + off[u]);
  }
}

// The launch reserves 32 KB of LDS that the kernel does not use, which
// holds a CU to five workgroups: fewer loads in flight at once, but
// workgroups that drift apart, so that stores overlap loads. Interleaved
// runs: A of 8192^3 65.7 -> 63.8 us, B of the decode shape 31.6 -> 31.1 us,
// A of the prefill shape unchanged; four per CU was as good on 8192^3 and
// slower elsewhere, two per CU 10-15% slower.
template <int G, int FMT, int IN, int U>
static hipError_t launch_rows_u(const QuantArgs& p, hipStream_t stream, int64_t nseg) {
  const int64_t per_wg = 4 * (64 / (G / InKind<IN>::kPerLoad)) * U;  // segments per workgroup of four waves
  hipLaunchKernelGGL((quant_fp8_rows<G, FMT, IN, U>), dim3((unsigned)((nseg + per_wg - 1) / per_wg)), dim3(256),
                     32u * 1024u, stream, p.x, p.q, p.scales, (unsigned)nseg, (int)p.cols);
  return hipGetLastError();
}

// Loads per lane: the most of 8, 4, 2 and 1 that still give at least 2048
// workgroups (eight per CU), else 1. Large operands keep eight loads in
// flight per lane; a small activation is spread over the whole chip instead
// of a few CUs. Interleaved runs, per-row factors at g = 128: A of the decode
// shape (64 x 7168, 28 workgroups at eight loads) 5.15 -> 2.52 us in FP32 and
// 5.15 -> 2.42 us in BF16 at one load; A of the prefill shape in BF16 (4096 x
// 2048) 10.1 -> 8.4 us at two (9.3 at one or four); A of 8192^3 in BF16 best
// at eight or four (44.3 us; two 46.4, one 56.5).
template <int G, int FMT, int IN>
static hipError_t launch_rows_g(const QuantArgs& p, hipStream_t stream) {
  const int64_t nseg = p.rows * (p.cols / G);
  constexpr int64_t per_load = 4 * (64 / (G / InKind<IN>::kPerLoad));  // segments per workgroup and load
  constexpr int64_t kMinGroups = 2048;
  if (nseg >= kMinGroups * per_load * 8) return launch_rows_u<G, FMT, IN, 8>(p, stream, nseg);
  if (nseg >= kMinGroups * per_load * 4) return launch_rows_u<G, FMT, IN, 4>(p, stream, nseg);
  if (nseg >= kMinGroups * per_load * 2) return launch_rows_u<G, FMT, IN, 2>(p, stream, nseg);
  return launch_rows_u<G, FMT, IN, 1>(p, stream, nseg);
}

template <int FMT, int IN>
static hipError_t launch_rows_f(const QuantArgs& p, hipStream_t stream) {
  switch (p.gran) {
    case 64: return launch_rows_g<64, FMT, IN>(p, stream);
    case 128: return launch_rows_g<128, FMT, IN>(p, stream);
    case 256: return launch_rows_g<256, FMT, IN>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int IN>
static hipError_t launch_rows_i(const QuantArgs& p, hipStream_t stream) {
  return p.fmt == 1 ? launch_rows_f<1, IN>(p, stream) : launch_rows_f<0, IN>(p, stream);
}

hipError_t launch_quant_rows(const QuantArgs& p, hipStream_t stream) {
  switch (p.in) {
    case 0: return launch_rows_i<0>(p, stream);
    case 1: return launch_rows_i<1>(p, stream);
    case 2: return launch_rows_i<2>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// For FP32 blocks of g = 128 (64 KB of input each) and at least four blocks
// per CU, the launch reserves 64 KB of LDS that the kernel does not use, so
// that two workgroups share a CU instead of five. Fewer blocks in flight at
// once stagger the workgroups: one block's stores overlap the next blocks'
// loads instead of every CU loading, then dividing, then storing together.
// Interleaved runs: B of the decode shape (1792 blocks) 30.7 -> 29.6 us, A of
// 8192^3 (4096 blocks) 61.0 -> 59.9 us; B of the prefill shape (896 blocks)
// was 2% slower this way (1.75 rounds of two per CU) and keeps five.
// Smaller blocks need every workgroup the registers allow, since two of them
// per CU hold too few bytes in flight: without the reservation FP32 g = 64
// ran 1.7-1.9x faster (B of the long-K shape 119.6 -> 64.5 us, A of 8192^3
// at g = 64 122.9 -> 65.7 us) and 16-bit g = 128 blocks (32 KB) 7-9% faster
// (A of 8192^3 in BF16 42.8 -> 39.4 us), 16-bit g = 64 1.5x (A of the long-K
// shape 33.8 -> 22.3 us); a 32 KB reservation (five per CU) fell in between.
// g = 256 runs 1024-thread workgroups, two per CU already.
template <int G, int FMT, int IN, int NT>
static hipError_t launch_gt(const QuantArgs& p, hipStream_t stream, int64_t nblocks, unsigned lds) {
  hipLaunchKernelGGL((quant_fp8_blocks<G, FMT, IN, NT>), dim3((unsigned)nblocks), dim3(NT), lds, stream, p.x, p.q,
                     p.scales, (int)p.rows, (int)p.cols);
  return hipGetLastError();
}

// With at most 256 blocks (one per CU) a block's workgroup has the CU to
// itself, and up to 1024 threads take a quarter of the passes of 256 over it.
// Interleaved runs, A of the decode shape (64 x 7168): g = 64 in FP32 (112
// blocks) 4.05 -> 3.01 us, g = 128 in BF16 3.28 -> 3.14 us, but g = 128 in
// FP32 3.67 -> 3.84 us (its 64-row blocks leave half of 1024 lanes idle);
// A of the 256^3 shape (4 blocks) 4.43 -> 4.21 us.
template <int G, int FMT, int IN>
static hipError_t launch_g(const QuantArgs& p, hipStream_t stream) {
  const int64_t nblocks = ((p.rows + G - 1) / G) * (p.cols / G);
  if constexpr (G == 256) {
    return launch_gt<G, FMT, IN, 1024>(p, stream, nblocks, 0u);
  } else {
    constexpr int kLanes = (G / InKind<IN>::kPerLoad) * G;  // 16-byte pieces of a block
    if (nblocks <= 256) return launch_gt<G, FMT, IN, kLanes < 1024 ? kLanes : 1024>(p, stream, nblocks, 0u);
    // Blocks of 16 or 32 KB (FP32 at g = 64, 16-bit input at g = 128) take
    // 512 threads, two or four loads per lane: interleaved runs, A of the
    // long-K shape in FP32 35.2 -> 31.5 us, its B 63.7 -> 60.0 us, A of 8192^3
    // in BF16 40.4 -> 39.2 us, B of the prefill shape in BF16 13.9 -> 12.8 us.
    // 8 KB blocks (16-bit, g = 64) keep 256, one load per lane being too few
    // (A of the long-K shape in BF16 22.6 -> 26.6 us at 512); FP32 at g = 128
    // keeps 256 and the reservation below.
    if constexpr ((IN == 0 && G == 64) || (IN != 0 && G == 128)) {
      return launch_gt<G, FMT, IN, 512>(p, stream, nblocks, 0u);
    } else {
      const unsigned lds = IN == 0 && G == 128 && nblocks >= 4 * 256 ? 64u * 1024u : 0u;
      return launch_gt<G, FMT, IN, 256>(p, stream, nblocks, lds);
    }
  }
}

template <int FMT, int IN>
static hipError_t launch_f(const QuantArgs& p, hipStream_t stream) {
  switch (p.gran) {
    case 64: return launch_g<64, FMT, IN>(p, stream);
    case 128: return launch_g<128, FMT, IN>(p, stream);
    case 256: return launch_g<256, FMT, IN>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int IN>
static hipError_t launch_i(const QuantArgs& p, hipStream_t stream) {
  return p.fmt == 1 ? launch_f<1, IN>(p, stream) : launch_f<0, IN>(p, stream);
}

hipError_t launch_quant(const QuantArgs& p, hipStream_t stream) {
  switch (p.in) {
    case 0: return launch_i<0>(p, stream);
    case 1: return launch_i<1>(p, stream);
    case 2: return launch_i<2>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
