// Block quantiser FP32 -> E4M3FN with one FP32 scale per g x g block, for
// gfx950. It produces the GEMM's inputs: the pages place quantisation outside
// the GEMM, say that activations must be quantised online and that the
// granularity must equal the GEMM's (DeepGEMM实战 §4.4), and that one factor
// per block maps the block into FP8 range (§2.2) by dividing (§5.2).
//
// Per block: amax = max |x| over the elements present (edge blocks past the
// last row are partial), scale = amax / 448 (FP32, correctly rounded; 1.0 for
// an all-zero block), code = E4M3(x / scale) with a correctly rounded FP32
// divide and the hardware's round-to-nearest-even conversion. Because
// |x / scale| <= 448 up to one rounding, which still rounds to 448, no value
// can overflow the format.
//
// One workgroup of 256 threads per block. The block (64 KB for g = 128) stays
// in registers between the amax pass and the encode pass, so x is read from
// HBM once: the kernel is bound by HBM bandwidth (4 bytes in, 1 byte out per
// element).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "quant_e4m3.h"

namespace dg {

typedef float v4f __attribute__((ext_vector_type(4)));

template <int G>
__global__ __launch_bounds__(256) void quant_e4m3_blocks(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                         float* __restrict__ scales, int rows, int cols) {
  constexpr int NT = 256;
  constexpr int ROW_V4 = G / 4;              // float4 per block row
  constexpr int ROWS_PER_PASS = NT / ROW_V4;  // block rows covered by one pass
  constexpr int PASSES = G / ROWS_PER_PASS;
  __shared__ float red[NT / 64];

  const int ncb = cols / G;
  const int rb = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  const int t = threadIdx.x;
  const int rsub = t / ROW_V4, c4 = t % ROW_V4;
  const int col = cb * G + c4 * 4;

  v4f v[PASSES];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = rb * G + p * ROWS_PER_PASS + rsub;
    if (r < rows) {
      v[p] = *reinterpret_cast<const v4f*>(x + (int64_t)r * cols + col);
    } else {
      v[p] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    }
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[p].x), fabsf(v[p].y)), fmaxf(fabsf(v[p].z), fabsf(v[p].w))));
  }
  // max is exact and order-free: wave butterfly, then across the 4 waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (t == 0) scales[blockIdx.x] = scale;

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = rb * G + p * ROWS_PER_PASS + rsub;
    if (r < rows) {
      // v_cvt_pk_fp8_f32 packs two E4M3 codes into the low or high 16 bits.
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(v[p].x / scale, v[p].y / scale, 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(v[p].z / scale, v[p].w / scale, packed, true);
      *reinterpret_cast<int*>(q + (int64_t)r * cols + col) = packed;
    }
  }
}

template <int G>
static hipError_t launch_quant(const QuantArgs& p, hipStream_t stream) {
  const int64_t nblocks = ((p.rows + G - 1) / G) * (p.cols / G);
  hipLaunchKernelGGL((quant_e4m3_blocks<G>), dim3((unsigned)nblocks), dim3(256), 0, stream, p.x, p.q, p.scales,
                     (int)p.rows, (int)p.cols);
  return hipGetLastError();
}

hipError_t launch_quant_e4m3(const QuantArgs& p, hipStream_t stream) {
  return p.gran == 64 ? launch_quant<64>(p, stream) : launch_quant<128>(p, stream);
}

}  // namespace dg
