// dgo: plain CPU oracle for the block-scaled FP8 GEMM.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
// this file: only the tests, the package smoke check and the benchmark's
// CPU-baseline leg use it. It shares no code, header, table or constant with
// the HIP library; the two meet only in the tests, through the seeded inputs.
//
// What it computes, and from which passage of the pages:
//
//  * E4M3 decode/encode. The pages give the format only as "4 exponent bits,
//    3 mantissa bits" (DeepGEMM-style template article, §3.4; DeepGEMM in
//    practice / DeepGEMM实战, §2.2) and name torch.float8_e4m3fn as the input
//    type (DeepGEMM实战, §4.2). The reading taken is the OCP E4M3FN format that
//    type implements: bias 7, exponent field 0 holds subnormals m/8 * 2^-6,
//    largest finite value 0x7E = 448, codes 0x7F/0xFF are NaN, no infinity.
//
//  * Block quantisation, the step that feeds the GEMM (DeepGEMM实战 §2.2: one
//    factor per 128x128 block maps the block into FP8 range when quantising;
//    §4.4: quantisation happens outside the GEMM and must use the GEMM's
//    granularity; §5.2: divide when quantising, multiply when dequantising).
//    Per g x g block: amax over the elements present (edge blocks are
//    partial), scale = amax / 448 in FP32 (1.0 for an all-zero block, and
//    for a block so small that amax / 448 underflows to zero), and
//    each element becomes E4M3(x / scale), an FP32 divide followed by
//    round-to-nearest-even with saturation to +-448.
//
//  * The GEMM, C = A * B^T in the NT layout (DeepGEMM实战 §3.3, §4.2): A is
//    [M,K], B is [N,K], both K-contiguous. Each g-wide K segment kb is summed
//    on its own (§3.2: segments accumulated separately, then added) and then
//    restored with the product of its two block scales (§2.2):
//        P[i,j,kb] = sum_{k in kb} dec(A[i,k]) * dec(B[j,k])
//        ref[i,j]  = sum_kb (sa[i/g,kb] * sb[j/g,kb]) * P[i,j,kb]   (kb ascending)
//    in FP64. Every E4M3 value is an integer multiple of 2^-9 below 2^9, so a
//    product is a multiple of 2^-18 below 2^18 and a sum of up to 2^14 of
//    them stays below 2^53 units: P is exact in FP64 in any order. The only
//    roundings are the scale multiply and the segment sum.
//
//  * E5M2 and mixed formats, g = 256 (the variants the pages name beside the
//    default: DeepGEMM实战 §2.2 lists E4M3 and E5M2 as the two FP8 formats,
//    §3.1 discusses other scale granularities). E5M2 is read as the OCP E5M2
//    format torch.float8_e5m2 implements: bias 15, exponent field 0 holds
//    subnormals m/4 * 2^-14, largest finite value 0x7B = 57344, exponent
//    field 31 is infinity (m = 0) or NaN. Quantisation to E5M2 follows the
//    same block rule with 57344 in place of 448. With an E5M2 operand a
//    segment partial is no longer exact in FP64 in general (products span
//    more than 53 bits); its relative error stays below K * 2^-53 of the sum
//    of the products' magnitudes, far inside the GEMM tolerance.
//
//  * Epilogue (the template article, §2.3 and §6: an extension point before
//    the result is written back, e.g. bias add, ReLU, GELU):
//        y[i,j] = act(ref[i,j] + bias[j])
//    in FP64, act = identity, ReLU max(y, 0), or GELU y * Phi(y) =
//    0.5 * y * (1 + erf(y / sqrt(2))) (the exact form; the pages name GELU
//    without choosing an approximation).
//
//  * Per-row A scales (the DeepGEMM-style template article, §3.4: scale
//    factors per tensor or per channel, per channel the more accurate and the
//    one the method usually takes): A carries one factor per row and g-wide
//    K segment (1 x g blocks), B keeps its g x g blocks:
//        ref[i,j]  = sum_kb (sa[i,kb] * sb[j/g,kb]) * P[i,j,kb]
//    and the quantiser's 1 x g variant takes amax over one row's segment.
//
//  * Operand layouts (DeepGEMM实战 §3.3: A and B may each be stored
//    transposed; the product is the same). Layout code bit 1: A stored
//    [K][M] (A[i,k] at a[k*M + i]) instead of [M][K]; bit 0: B stored [K][N]
//    (B[j,k] at b[k*N + j]) instead of [N][K]. Codes: 0 = NT (the default),
//    1 = NN, 2 = TT, 3 = TN (first letter A, second B, as in C = op(A) op(B)
//    with op(B) = B^T for B stored [N][K]). The scales keep their logical
//    shapes: sa [ceil(M/g)][K/g], sb [ceil(N/g)][K/g].
//
//  * 16-bit inputs to the quantiser (DeepGEMM实战 §4.4: the weights and
//    activations that are quantised to FP8 arrive in FP16 or BF16). Such an
//    input is first decoded to its exact value, which FP32 holds exactly,
//    and the block rule above then applies unchanged. BF16 is read as the
//    format that keeps FP32's sign and 8-bit exponent (bias 127) and 7
//    fraction bits, FP16 as IEEE binary16 (5-bit exponent, bias 15, 10
//    fraction bits); both have subnormals at exponent field 0.
//
// Scale tensors are row-major FP32: sa is [ceil(M/g)][K/g] ([M][K/g] with
// per-row A scales), sb is [ceil(N/g)][K/g]. K must be a multiple of g.
//
// Build: g++ -O2 -std=c++17 -ffp-contract=off -fPIC -shared -pthread.
// No fast-math: the arithmetic above must be IEEE single/double as written.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// One worker per slice of [0, n). Plain std::thread fan-out.
template <typename F>
void parallel_for(int64_t n, int nthreads, F body) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) {
    body(0, n);
    return;
  }
  std::vector<std::thread> pool;
  int64_t per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = t * per, hi = lo + per < n ? lo + per : n;
    if (lo >= hi) break;
    pool.emplace_back(body, lo, hi);
  }
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// OCP E4M3FN decode of one code, straight from the bit fields.
double dgo_e4m3_decode(uint8_t code) {
  const int s = code >> 7;
  const int e = (code >> 3) & 0xF;
  const int m = code & 0x7;
  if (e == 0xF && m == 0x7) return std::nan("");
  double mag;
  if (e == 0)
    mag = std::ldexp((double)m / 8.0, -6);             // subnormal: m/8 * 2^(1-7)
  else
    mag = std::ldexp(1.0 + (double)m / 8.0, e - 7);    // normal: (1+m/8) * 2^(e-7)
  return s ? -mag : mag;
}

// FP32 -> E4M3FN: round to nearest, ties to even, saturate to +-448.
// Never produces NaN (finite input assumed).
uint8_t dgo_e4m3_encode(float y) {
  const uint8_t sign = std::signbit(y) ? 0x80 : 0x00;
  const double v = std::fabs((double)y);
  if (v >= 448.0) return sign | 0x7E;
  if (v < std::ldexp(1.0, -6)) {
    // Subnormal range, spacing 2^-9. Scaling by 512 is exact; nearbyint rounds
    // half to even in the default rounding mode. n == 8 is code 0x08 = 2^-6,
    // the smallest normal, so the code is n itself.
    const double n = std::nearbyint(v * 512.0);
    return sign | (uint8_t)n;
  }
  int e2;
  std::frexp(v, &e2);            // v = f * 2^e2, f in [0.5, 1)
  int E = e2 - 1;                // v in [2^E, 2^(E+1)), -6 <= E <= 8
  double n = std::nearbyint(std::ldexp(v, 3 - E));  // mantissa steps: n in [8, 16]
  if (n == 16.0) {               // rounded up into the next binade
    n = 8.0;
    E += 1;
  }
  return sign | (uint8_t)(((E + 7) << 3) | ((int)n - 8));
}

// OCP E5M2 decode of one code, straight from the bit fields.
double dgo_e5m2_decode(uint8_t code) {
  const int s = code >> 7;
  const int e = (code >> 2) & 0x1F;
  const int m = code & 0x3;
  double mag;
  if (e == 0x1F)
    mag = m == 0 ? INFINITY : std::nan("");
  else if (e == 0)
    mag = std::ldexp((double)m / 4.0, -14);            // subnormal: m/4 * 2^(1-15)
  else
    mag = std::ldexp(1.0 + (double)m / 4.0, e - 15);   // normal: (1+m/4) * 2^(e-15)
  return s ? -mag : mag;
}

// FP32 -> E5M2: round to nearest, ties to even, saturate to +-57344.
// Never produces infinity or NaN (finite input assumed).
uint8_t dgo_e5m2_encode(float y) {
  const uint8_t sign = std::signbit(y) ? 0x80 : 0x00;
  const double v = std::fabs((double)y);
  if (v >= 57344.0) return sign | 0x7B;
  if (v < std::ldexp(1.0, -14)) {
    // Subnormal range, spacing 2^-16; n == 4 is code 0x04 = 2^-14, the
    // smallest normal, so the code is n itself.
    const double n = std::nearbyint(v * 65536.0);
    return sign | (uint8_t)n;
  }
  int e2;
  std::frexp(v, &e2);
  int E = e2 - 1;                                     // v in [2^E, 2^(E+1)), -14 <= E <= 15
  double n = std::nearbyint(std::ldexp(v, 2 - E));    // mantissa steps: n in [4, 8]
  if (n == 8.0) {
    n = 4.0;
    E += 1;
  }
  return sign | (uint8_t)(((E + 15) << 2) | ((int)n - 4));
}

// Format codes shared with the Python side: 0 = E4M3FN, 1 = E5M2.
// A block's factor: amax / fmax in FP32, or 1.0 where that is zero: for an
// all-zero block, and for a block whose amax is so small (below fmax times
// half the smallest FP32 subnormal) that the quotient underflows to zero; a
// zero factor would divide by zero, while 1.0 encodes such a block's values
// (all below fmax * 2^-150, under 2^-134 in magnitude) as zeros.
static float block_scale(float amax, float fmax) {
  const float s = amax / fmax;
  return s > 0.0f ? s : 1.0f;
}

static double decode_fmt(int fmt, uint8_t code) { return fmt == 1 ? dgo_e5m2_decode(code) : dgo_e4m3_decode(code); }
static uint8_t encode_fmt(int fmt, float y) { return fmt == 1 ? dgo_e5m2_encode(y) : dgo_e4m3_encode(y); }

void dgo_e5m2_decode_n(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = dgo_e5m2_decode(codes[i]);
}

void dgo_e5m2_encode_n(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = dgo_e5m2_encode(y[i]);
}

// Decode an array of codes (convenience for the Python side).
void dgo_e4m3_decode_n(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = dgo_e4m3_decode(codes[i]);
}

void dgo_e4m3_encode_n(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = dgo_e4m3_encode(y[i]);
}

// Block quantiser. x is [rows][cols] FP32 row-major; q receives [rows][cols]
// E4M3 codes; scales receives [ceil(rows/g)][cols/g] FP32.
// Returns 0, or -1 on bad arguments.
int dgo_quantize_blocks(const float* x, int64_t rows, int64_t cols, int g, uint8_t* q,
                        float* scales, int nthreads) {
  if (!x || !q || !scales || rows <= 0 || cols <= 0 || g <= 0 || cols % g != 0) return -1;
  const int64_t nrb = (rows + g - 1) / g, ncb = cols / g;
  parallel_for(nrb, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t rb = lo; rb < hi; ++rb) {
      const int64_t r0 = rb * g, r1 = (r0 + g < rows) ? r0 + g : rows;
      for (int64_t cb = 0; cb < ncb; ++cb) {
        const int64_t c0 = cb * g, c1 = c0 + g;
        float amax = 0.0f;
        for (int64_t r = r0; r < r1; ++r)
          for (int64_t c = c0; c < c1; ++c) {
            const float a = std::fabs(x[r * cols + c]);
            if (a > amax) amax = a;
          }
        const float scale = block_scale(amax, 448.0f);
        scales[rb * ncb + cb] = scale;
        for (int64_t r = r0; r < r1; ++r)
          for (int64_t c = c0; c < c1; ++c) q[r * cols + c] = dgo_e4m3_encode(x[r * cols + c] / scale);
      }
    }
  });
  return 0;
}

// Segment partials P[kb] = sum_{k in segment kb} dec(a_row[k]) * dec(b_row[k])
// for one output element (a_row = A[i,:], b_row = B[j,:]), FP64.
void dgo_segment_partials(const uint8_t* a_row, const uint8_t* b_row, int64_t K, int g, double* P) {
  double tab[256];
  for (int c = 0; c < 256; ++c) tab[c] = dgo_e4m3_decode((uint8_t)c);
  for (int64_t kb = 0; kb < K / g; ++kb) {
    double p = 0.0;
    for (int64_t k = kb * g; k < kb * g + g; ++k) p += tab[a_row[k]] * tab[b_row[k]];
    P[kb] = p;
  }
}

// Reference GEMM in FP64 on a subset of the output.
//   rows: nrows row indices into [0,M) (NULL = all M rows, nrows ignored)
//   cols: ncols column indices into [0,N) (NULL = all N columns)
//   out : [nrows][ncols] FP64, out[r][c] = ref[rows[r], cols[c]]
// Returns 0, or -1 on bad arguments.
int dgo_gemm_ref(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M,
                 int64_t N, int64_t K, int g, const int64_t* rows, int64_t nrows, const int64_t* cols,
                 int64_t ncols, double* out, int nthreads) {
  if (!a || !b || !sa || !sb || !out || M <= 0 || N <= 0 || K <= 0 || g <= 0 || K % g != 0) return -1;
  if (!rows) nrows = M;
  if (!cols) ncols = N;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -1;
  for (int64_t c = 0; cols && c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= N) return -1;

  double tab[256];
  for (int c = 0; c < 256; ++c) tab[c] = dgo_e4m3_decode((uint8_t)c);
  const int64_t nkb = K / g;

  parallel_for(nrows, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t r = lo; r < hi; ++r) {
      const int64_t i = rows ? rows[r] : r;
      const uint8_t* arow = a + i * K;
      const float* sarow = sa + (i / g) * nkb;
      for (int64_t c = 0; c < ncols; ++c) {
        const int64_t j = cols ? cols[c] : c;
        const uint8_t* brow = b + j * K;
        const float* sbrow = sb + (j / g) * nkb;
        double ref = 0.0;
        for (int64_t kb = 0; kb < nkb; ++kb) {
          double p = 0.0;  // exact: see the header
          for (int64_t k = kb * g; k < kb * g + g; ++k) p += tab[arow[k]] * tab[brow[k]];
          const double s = (double)sarow[kb] * (double)sbrow[kb];  // exact (24 x 24 bits)
          ref += s * p;
        }
        out[r * ncols + c] = ref;
      }
    }
  });
  return 0;
}

// Block quantiser for either format: as dgo_quantize_blocks with the
// format's largest finite value (448 for E4M3, 57344 for E5M2) in the scale.
int dgo_quantize_blocks_fmt(const float* x, int64_t rows, int64_t cols, int g, int fmt, uint8_t* q,
                            float* scales, int nthreads) {
  if (!x || !q || !scales || rows <= 0 || cols <= 0 || g <= 0 || cols % g != 0 || (fmt != 0 && fmt != 1)) return -1;
  const float fmax = fmt == 1 ? 57344.0f : 448.0f;
  const int64_t nrb = (rows + g - 1) / g, ncb = cols / g;
  parallel_for(nrb, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t rb = lo; rb < hi; ++rb) {
      const int64_t r0 = rb * g, r1 = (r0 + g < rows) ? r0 + g : rows;
      for (int64_t cb = 0; cb < ncb; ++cb) {
        const int64_t c0 = cb * g, c1 = c0 + g;
        float amax = 0.0f;
        for (int64_t r = r0; r < r1; ++r)
          for (int64_t c = c0; c < c1; ++c) {
            const float a = std::fabs(x[r * cols + c]);
            if (a > amax) amax = a;
          }
        const float scale = block_scale(amax, fmax);
        scales[rb * ncb + cb] = scale;
        for (int64_t r = r0; r < r1; ++r)
          for (int64_t c = c0; c < c1; ++c) q[r * cols + c] = encode_fmt(fmt, x[r * cols + c] / scale);
      }
    }
  });
  return 0;
}

// Reference GEMM with the operands' formats given (fmt_a, fmt_b: 0 = E4M3,
// 1 = E5M2); otherwise exactly dgo_gemm_ref.
int dgo_gemm_ref_fmt(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M,
                     int64_t N, int64_t K, int g, int fmt_a, int fmt_b, const int64_t* rows, int64_t nrows,
                     const int64_t* cols, int64_t ncols, double* out, int nthreads) {
  if (!a || !b || !sa || !sb || !out || M <= 0 || N <= 0 || K <= 0 || g <= 0 || K % g != 0) return -1;
  if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1)) return -1;
  if (!rows) nrows = M;
  if (!cols) ncols = N;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -1;
  for (int64_t c = 0; cols && c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= N) return -1;

  double ta[256], tb[256];
  for (int c = 0; c < 256; ++c) {
    ta[c] = decode_fmt(fmt_a, (uint8_t)c);
    tb[c] = decode_fmt(fmt_b, (uint8_t)c);
  }
  const int64_t nkb = K / g;

  parallel_for(nrows, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t r = lo; r < hi; ++r) {
      const int64_t i = rows ? rows[r] : r;
      const uint8_t* arow = a + i * K;
      const float* sarow = sa + (i / g) * nkb;
      for (int64_t c = 0; c < ncols; ++c) {
        const int64_t j = cols ? cols[c] : c;
        const uint8_t* brow = b + j * K;
        const float* sbrow = sb + (j / g) * nkb;
        double ref = 0.0;
        for (int64_t kb = 0; kb < nkb; ++kb) {
          double p = 0.0;
          for (int64_t k = kb * g; k < kb * g + g; ++k) p += ta[arow[k]] * tb[brow[k]];
          const double s = (double)sarow[kb] * (double)sbrow[kb];
          ref += s * p;
        }
        out[r * ncols + c] = ref;
      }
    }
  });
  return 0;
}

// Quantiser with 1 x g blocks (one factor per row and g-wide column segment):
// scales receives [rows][cols/g]; otherwise as dgo_quantize_blocks_fmt.
int dgo_quantize_rows_fmt(const float* x, int64_t rows, int64_t cols, int g, int fmt, uint8_t* q, float* scales,
                          int nthreads) {
  if (!x || !q || !scales || rows <= 0 || cols <= 0 || g <= 0 || cols % g != 0 || (fmt != 0 && fmt != 1)) return -1;
  const float fmax = fmt == 1 ? 57344.0f : 448.0f;
  const int64_t ncb = cols / g;
  parallel_for(rows, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t r = lo; r < hi; ++r)
      for (int64_t cb = 0; cb < ncb; ++cb) {
        const float* seg = x + r * cols + cb * g;
        float amax = 0.0f;
        for (int64_t c = 0; c < g; ++c)
          if (std::fabs(seg[c]) > amax) amax = std::fabs(seg[c]);
        const float scale = block_scale(amax, fmax);
        scales[r * ncb + cb] = scale;
        for (int64_t c = 0; c < g; ++c) q[r * cols + cb * g + c] = encode_fmt(fmt, seg[c] / scale);
      }
  });
  return 0;
}

// Reference GEMM with per-row A scales: sa is [M][K/g] (one factor per row of
// A and K segment), sb is [ceil(N/g)][K/g]; formats as dgo_gemm_ref_fmt.
//   ref[i,j] = sum_kb (sa[i,kb] * sb[j/g,kb]) * P[i,j,kb]   (kb ascending)
int dgo_gemm_ref_rowa(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M, int64_t N,
                      int64_t K, int g, int fmt_a, int fmt_b, const int64_t* rows, int64_t nrows,
                      const int64_t* cols, int64_t ncols, double* out, int nthreads) {
  if (!a || !b || !sa || !sb || !out || M <= 0 || N <= 0 || K <= 0 || g <= 0 || K % g != 0) return -1;
  if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1)) return -1;
  if (!rows) nrows = M;
  if (!cols) ncols = N;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -1;
  for (int64_t c = 0; cols && c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= N) return -1;

  double ta[256], tb[256];
  for (int c = 0; c < 256; ++c) {
    ta[c] = decode_fmt(fmt_a, (uint8_t)c);
    tb[c] = decode_fmt(fmt_b, (uint8_t)c);
  }
  const int64_t nkb = K / g;

  parallel_for(nrows, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t r = lo; r < hi; ++r) {
      const int64_t i = rows ? rows[r] : r;
      const uint8_t* arow = a + i * K;
      const float* sarow = sa + i * nkb;  // this row's own factors
      for (int64_t c = 0; c < ncols; ++c) {
        const int64_t j = cols ? cols[c] : c;
        const uint8_t* brow = b + j * K;
        const float* sbrow = sb + (j / g) * nkb;
        double ref = 0.0;
        for (int64_t kb = 0; kb < nkb; ++kb) {
          double p = 0.0;
          for (int64_t k = kb * g; k < kb * g + g; ++k) p += ta[arow[k]] * tb[brow[k]];
          const double s = (double)sarow[kb] * (double)sbrow[kb];
          ref += s * p;
        }
        out[r * ncols + c] = ref;
      }
    }
  });
  return 0;
}

// Reference GEMM with the operands in any of the four layouts (see the
// header): the same sums as dgo_gemm_ref_fmt, each element read from where
// the layout stores it.
int dgo_gemm_ref_layout(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M, int64_t N,
                        int64_t K, int g, int layout, int fmt_a, int fmt_b, const int64_t* rows, int64_t nrows,
                        const int64_t* cols, int64_t ncols, double* out, int nthreads) {
  if (!a || !b || !sa || !sb || !out || M <= 0 || N <= 0 || K <= 0 || g <= 0 || K % g != 0) return -1;
  if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1) || layout < 0 || layout > 3) return -1;
  if (!rows) nrows = M;
  if (!cols) ncols = N;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -1;
  for (int64_t c = 0; cols && c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= N) return -1;
  const bool a_km = (layout & 2) != 0, b_kn = (layout & 1) != 0;

  double ta[256], tb[256];
  for (int c = 0; c < 256; ++c) {
    ta[c] = decode_fmt(fmt_a, (uint8_t)c);
    tb[c] = decode_fmt(fmt_b, (uint8_t)c);
  }
  const int64_t nkb = K / g;

  parallel_for(nrows, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t r = lo; r < hi; ++r) {
      const int64_t i = rows ? rows[r] : r;
      const float* sarow = sa + (i / g) * nkb;
      for (int64_t c = 0; c < ncols; ++c) {
        const int64_t j = cols ? cols[c] : c;
        const float* sbrow = sb + (j / g) * nkb;
        double ref = 0.0;
        for (int64_t kb = 0; kb < nkb; ++kb) {
          double p = 0.0;
          for (int64_t k = kb * g; k < kb * g + g; ++k) {
            const uint8_t ca = a_km ? a[k * M + i] : a[i * K + k];
            const uint8_t cb = b_kn ? b[k * N + j] : b[j * K + k];
            p += ta[ca] * tb[cb];
          }
          const double s = (double)sarow[kb] * (double)sbrow[kb];
          ref += s * p;
        }
        out[r * ncols + c] = ref;
      }
    }
  });
  return 0;
}

// Epilogue on an oracle result in place: ref is [nrows][ncols] for output
// columns cols (NULL = 0..ncols-1); bias is FP32 [N] or NULL; act 0 = none,
// 1 = ReLU, 2 = GELU (erf form). Returns 0, or -1 on bad arguments.
int dgo_epilogue(double* ref, int64_t nrows, int64_t ncols, const int64_t* cols, const float* bias, int act) {
  if (!ref || nrows < 0 || ncols < 0 || act < 0 || act > 2) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    for (int64_t c = 0; c < ncols; ++c) {
      const int64_t j = cols ? cols[c] : c;
      double y = ref[r * ncols + c] + (bias ? (double)bias[j] : 0.0);
      if (act == 1) y = y > 0.0 ? y : 0.0;
      if (act == 2) y = 0.5 * y * (1.0 + std::erf(y / std::sqrt(2.0)));
      ref[r * ncols + c] = y;
    }
  return 0;
}

// BF16 decode of one bit pattern from its fields: sign, 8-bit exponent
// (bias 127), 7-bit fraction; exponent 0 holds subnormals f/128 * 2^-126,
// exponent 255 infinity (f = 0) or NaN.
double dgo_bf16_decode(uint16_t bits) {
  const int s = bits >> 15;
  const int e = (bits >> 7) & 0xFF;
  const int f = bits & 0x7F;
  double mag;
  if (e == 0xFF)
    mag = f ? std::nan("") : HUGE_VAL;
  else if (e == 0)
    mag = std::ldexp((double)f / 128.0, -126);
  else
    mag = std::ldexp(1.0 + (double)f / 128.0, e - 127);
  return s ? -mag : mag;
}

// IEEE binary16 decode of one bit pattern: sign, 5-bit exponent (bias 15),
// 10-bit fraction; exponent 0 holds subnormals f/1024 * 2^-14, exponent 31
// infinity (f = 0) or NaN.
double dgo_f16_decode(uint16_t bits) {
  const int s = bits >> 15;
  const int e = (bits >> 10) & 0x1F;
  const int f = bits & 0x3FF;
  double mag;
  if (e == 0x1F)
    mag = f ? std::nan("") : HUGE_VAL;
  else if (e == 0)
    mag = std::ldexp((double)f / 1024.0, -14);
  else
    mag = std::ldexp(1.0 + (double)f / 1024.0, e - 15);
  return s ? -mag : mag;
}

// Decode n 16-bit patterns (kind 1 = BF16, 2 = FP16) to FP32. Every finite
// value of either format is exactly an FP32 value, so the narrowing from the
// FP64 decode is exact. Returns 0, or -1 for an unknown kind.
int dgo_decode16_n(const uint16_t* bits, int64_t n, int kind, float* out) {
  if (kind != 1 && kind != 2) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(kind == 1 ? dgo_bf16_decode(bits[i]) : dgo_f16_decode(bits[i]));
  return 0;
}

int dgo_hardware_threads(void) {
  unsigned n = std::thread::hardware_concurrency();
  return n ? (int)n : 1;
}

}  // extern "C"
