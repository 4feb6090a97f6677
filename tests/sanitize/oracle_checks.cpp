// The oracle's C++ (oracle/dgo.cpp) on small inputs under AddressSanitizer and
// UndefinedBehaviorSanitizer, built for the CPU by tests/test_sanitize.py:
// every exported function on ragged shapes, subsets of rows and columns, one
// and several threads, and the argument errors it must reject. Any
// out-of-bounds access, use of freed memory, leak or undefined operation ends
// the run with the sanitizer's report; the checks below add the equalities
// that hold exactly between the oracle's own functions (the same sums in the
// same order), so a run that only touches memory correctly but mixes up an
// index still fails. Exit status 0 when everything holds.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

extern "C" {
double dgo_e4m3_decode(uint8_t code);
uint8_t dgo_e4m3_encode(float y);
double dgo_e5m2_decode(uint8_t code);
uint8_t dgo_e5m2_encode(float y);
void dgo_e4m3_decode_n(const uint8_t* codes, int64_t n, double* out);
void dgo_e4m3_encode_n(const float* y, int64_t n, uint8_t* out);
void dgo_e5m2_decode_n(const uint8_t* codes, int64_t n, double* out);
void dgo_e5m2_encode_n(const float* y, int64_t n, uint8_t* out);
int dgo_quantize_blocks(const float* x, int64_t rows, int64_t cols, int g, uint8_t* q, float* scales, int nthreads);
int dgo_quantize_blocks_fmt(const float* x, int64_t rows, int64_t cols, int g, int fmt, uint8_t* q, float* scales,
                            int nthreads);
int dgo_quantize_rows_fmt(const float* x, int64_t rows, int64_t cols, int g, int fmt, uint8_t* q, float* scales,
                          int nthreads);
void dgo_segment_partials(const uint8_t* a_row, const uint8_t* b_row, int64_t K, int g, double* P);
int dgo_gemm_ref(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M, int64_t N,
                 int64_t K, int g, const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                 double* out, int nthreads);
int dgo_gemm_ref_fmt(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M, int64_t N,
                     int64_t K, int g, int fmt_a, int fmt_b, const int64_t* rows, int64_t nrows, const int64_t* cols,
                     int64_t ncols, double* out, int nthreads);
int dgo_gemm_ref_rowa(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M, int64_t N,
                      int64_t K, int g, int fmt_a, int fmt_b, const int64_t* rows, int64_t nrows,
                      const int64_t* cols, int64_t ncols, double* out, int nthreads);
int dgo_gemm_ref_layout(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb, int64_t M, int64_t N,
                        int64_t K, int g, int layout, int fmt_a, int fmt_b, const int64_t* rows, int64_t nrows,
                        const int64_t* cols, int64_t ncols, double* out, int nthreads);
int dgo_epilogue(double* ref, int64_t nrows, int64_t ncols, const int64_t* cols, const float* bias, int act);
int dgo_hardware_threads(void);
}

namespace {

int g_failures = 0;

void check(bool ok, const char* what, long long a = 0, long long b = 0, long long c = 0) {
  if (!ok) {
    ++g_failures;
    std::fprintf(stderr, "FAILED: %s (%lld, %lld, %lld)\n", what, a, b, c);
  }
}

// xorshift64: test data only
struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  uint64_t next() {
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return s;
  }
  float normal() {  // sum of uniforms: rough bell, plenty for these checks
    double t = 0;
    for (int i = 0; i < 4; ++i) t += (double)(next() >> 11) * (1.0 / 9007199254740992.0);
    return (float)((t - 2.0) * 1.7);
  }
};

bool same_bits(double x, double y) { return std::memcmp(&x, &y, sizeof x) == 0; }

void codecs() {
  // every code decodes; finite codes survive encode(decode(c)) exactly
  std::vector<uint8_t> codes(256), back(256);
  std::vector<double> d4(256), d5(256);
  std::vector<float> f(256);
  for (int c = 0; c < 256; ++c) codes[c] = (uint8_t)c;
  dgo_e4m3_decode_n(codes.data(), 256, d4.data());
  dgo_e5m2_decode_n(codes.data(), 256, d5.data());
  for (int c = 0; c < 256; ++c) {
    check(same_bits(d4[c], dgo_e4m3_decode((uint8_t)c)) || (std::isnan(d4[c]) && std::isnan(dgo_e4m3_decode((uint8_t)c))),
          "e4m3 decode_n", c);
    if (std::isfinite(d4[c]) && d4[c] != 0.0) check(d4[c] == dgo_e4m3_decode(dgo_e4m3_encode((float)d4[c])), "e4m3 round trip", c);
    if (std::isfinite(d5[c]) && d5[c] != 0.0) check(d5[c] == dgo_e5m2_decode(dgo_e5m2_encode((float)d5[c])), "e5m2 round trip", c);
    f[c] = std::isfinite(d4[c]) ? (float)d4[c] : 0.0f;
  }
  dgo_e4m3_encode_n(f.data(), 256, back.data());
  for (int c = 0; c < 256; ++c)
    if (std::isfinite(d4[c]) && d4[c] != 0.0) check(back[c] == codes[c], "e4m3 encode_n", c);
  dgo_e5m2_encode_n(f.data(), 256, back.data());
  // edge values (the encoders take finite inputs): saturation, signed zero,
  // subnormals, the largest finite floats
  const float edge[] = {0.0f, -0.0f, 1e-30f, -1e-30f, 0.0009765625f, 448.0f, 464.0f, 1e30f, -1e30f,
                        57344.0f, 61440.0f, 1.5258789e-05f, 3.4028235e38f, -3.4028235e38f};
  for (float y : edge) {
    (void)dgo_e4m3_decode(dgo_e4m3_encode(y));
    (void)dgo_e5m2_decode(dgo_e5m2_encode(y));
  }
  check(dgo_e4m3_decode(dgo_e4m3_encode(1e30f)) == 448.0, "e4m3 saturates");
  check(dgo_e5m2_decode(dgo_e5m2_encode(1e30f)) == 57344.0, "e5m2 saturates");
}

// quantisers on a ragged shape: exact-size buffers, every block written once
void quantisers(int64_t rows, int64_t cols, int g, int nthreads, uint64_t seed) {
  Rng r(seed);
  std::vector<float> x((size_t)(rows * cols));
  for (auto& v : x) v = r.normal();
  // one all-zero block when there is room for it
  for (int64_t i = 0; i < rows && i < g; ++i)
    for (int64_t j = 0; j < g && j < cols; ++j) x[(size_t)(i * cols + j)] = 0.0f;
  const int64_t nrb = (rows + g - 1) / g, ncb = cols / g;
  std::vector<uint8_t> q((size_t)(rows * cols)), q2((size_t)(rows * cols));
  std::vector<float> s((size_t)(nrb * ncb)), s2((size_t)(nrb * ncb)), sr((size_t)(rows * ncb));
  check(dgo_quantize_blocks(x.data(), rows, cols, g, q.data(), s.data(), nthreads) == 0, "quantize_blocks", rows, cols, g);
  check(dgo_quantize_blocks_fmt(x.data(), rows, cols, g, 0, q2.data(), s2.data(), 1) == 0, "quantize_blocks_fmt", rows, cols, g);
  check(q == q2 && s == s2, "blocks: E4M3 through both quantisers, any thread count", rows, cols, g);
  check(s[0] == 1.0f, "all-zero block has factor 1", rows, cols, g);
  check(dgo_quantize_blocks_fmt(x.data(), rows, cols, g, 1, q2.data(), s2.data(), nthreads) == 0, "quantize e5m2");
  check(dgo_quantize_rows_fmt(x.data(), rows, cols, g, 0, q2.data(), sr.data(), nthreads) == 0, "quantize_rows");
  // dequantised values stay within half an E4M3 step of the input
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j) {
      const double v = dgo_e4m3_decode(q2[(size_t)(i * cols + j)]) * sr[(size_t)(i * ncb + j / g)];
      check(std::fabs(v - x[(size_t)(i * cols + j)]) <= std::fabs(x[(size_t)(i * cols + j)]) * 0.0625 + 1e-30 + sr[(size_t)(i * ncb + j / g)] * 0.001953125,
            "rows quantiser error", i, j);
    }
}

void gemms(int64_t M, int64_t N, int64_t K, int g, int nthreads, uint64_t seed) {
  Rng r(seed);
  std::vector<uint8_t> a((size_t)(M * K)), b((size_t)(N * K));
  for (auto& v : a) {
    v = (uint8_t)r.next();
    if ((v & 0x7F) == 0x7F) v ^= 1;  // no E4M3 NaN
    if ((v & 0x7C) == 0x7C) v &= 0xF3;  // no E5M2 inf/NaN either
  }
  for (auto& v : b) {
    v = (uint8_t)r.next();
    if ((v & 0x7F) == 0x7F) v ^= 1;
    if ((v & 0x7C) == 0x7C) v &= 0xF3;
  }
  const int64_t nkb = K / g, mb = (M + g - 1) / g, nb = (N + g - 1) / g;
  std::vector<float> sa((size_t)(mb * nkb)), sb((size_t)(nb * nkb)), sar((size_t)(M * nkb));
  for (auto& v : sa) v = std::ldexp(1.0f + (float)(r.next() % 64) / 64.0f, (int)(r.next() % 9) - 4);
  for (auto& v : sb) v = std::ldexp(1.0f + (float)(r.next() % 64) / 64.0f, (int)(r.next() % 9) - 4);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t kb = 0; kb < nkb; ++kb) sar[(size_t)(i * nkb + kb)] = sa[(size_t)((i / g) * nkb + kb)];

  std::vector<double> full((size_t)(M * N)), full2((size_t)(M * N));
  check(dgo_gemm_ref(a.data(), b.data(), sa.data(), sb.data(), M, N, K, g, nullptr, 0, nullptr, 0, full.data(),
                     nthreads) == 0, "gemm_ref", M, N, K);
  check(dgo_gemm_ref_fmt(a.data(), b.data(), sa.data(), sb.data(), M, N, K, g, 0, 0, nullptr, 0, nullptr, 0,
                         full2.data(), 1) == 0, "gemm_ref_fmt", M, N, K);
  check(full == full2, "gemm_ref and gemm_ref_fmt(E4M3) agree exactly", M, N, K);
  check(dgo_gemm_ref_rowa(a.data(), b.data(), sar.data(), sb.data(), M, N, K, g, 0, 0, nullptr, 0, nullptr, 0,
                          full2.data(), nthreads) == 0, "gemm_ref_rowa", M, N, K);
  check(full == full2, "per-row factors equal to the block's give the block result", M, N, K);

  // transposed stores through the layout reference: the same sums
  std::vector<uint8_t> at((size_t)(M * K)), bt((size_t)(N * K));
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) at[(size_t)(k * M + i)] = a[(size_t)(i * K + k)];
  for (int64_t j = 0; j < N; ++j)
    for (int64_t k = 0; k < K; ++k) bt[(size_t)(k * N + j)] = b[(size_t)(j * K + k)];
  for (int layout = 0; layout < 4; ++layout) {
    const uint8_t* as = (layout & 2) ? at.data() : a.data();
    const uint8_t* bs = (layout & 1) ? bt.data() : b.data();
    check(dgo_gemm_ref_layout(as, bs, sa.data(), sb.data(), M, N, K, g, layout, 0, 0, nullptr, 0, nullptr, 0,
                              full2.data(), nthreads) == 0, "gemm_ref_layout", layout);
    check(full == full2, "every layout gives the NT sums", layout, M, N);
  }
  for (int fa = 0; fa < 2; ++fa)
    for (int fb = 0; fb < 2; ++fb)
      check(dgo_gemm_ref_fmt(a.data(), b.data(), sa.data(), sb.data(), M, N, K, g, fa, fb, nullptr, 0, nullptr, 0,
                             full2.data(), nthreads) == 0, "gemm_ref_fmt formats", fa, fb);

  // a subset of rows and columns (repeats and the last index included)
  std::vector<int64_t> rows = {M - 1, 0, M / 2, M - 1}, cols = {N - 1, N / 3, 0};
  std::vector<double> sub(rows.size() * cols.size());
  check(dgo_gemm_ref(a.data(), b.data(), sa.data(), sb.data(), M, N, K, g, rows.data(), (int64_t)rows.size(),
                     cols.data(), (int64_t)cols.size(), sub.data(), nthreads) == 0, "gemm_ref subset");
  for (size_t i = 0; i < rows.size(); ++i)
    for (size_t j = 0; j < cols.size(); ++j)
      check(same_bits(sub[i * cols.size() + j], full[(size_t)(rows[i] * N + cols[j])]), "subset matches", (long long)i,
            (long long)j);

  // one element from its segment partials, summed in segment order
  std::vector<double> P((size_t)nkb);
  const int64_t i0 = M - 1, j0 = N / 3;
  dgo_segment_partials(a.data() + i0 * K, b.data() + j0 * K, K, g, P.data());
  double e = 0.0;
  for (int64_t kb = 0; kb < nkb; ++kb)
    e += ((double)sa[(size_t)((i0 / g) * nkb + kb)] * (double)sb[(size_t)((j0 / g) * nkb + kb)]) * P[(size_t)kb];
  check(same_bits(e, full[(size_t)(i0 * N + j0)]), "segment partials rebuild the element");

  // epilogue on the subset, with and without bias
  std::vector<float> bias((size_t)N);
  for (auto& v : bias) v = r.normal();
  for (int act = 0; act < 3; ++act) {
    std::vector<double> y = sub;
    check(dgo_epilogue(y.data(), (int64_t)rows.size(), (int64_t)cols.size(), cols.data(), bias.data(), act) == 0,
          "epilogue", act);
    std::vector<double> z = sub;
    check(dgo_epilogue(z.data(), (int64_t)rows.size(), (int64_t)cols.size(), cols.data(), nullptr, act) == 0,
          "epilogue without bias", act);
    if (act == 1)
      for (double v : y) check(v >= 0.0, "ReLU is non-negative");
  }
}

void rejects() {
  uint8_t a[256] = {}, b[256] = {}, q[256] = {};
  float sa[4] = {1, 1, 1, 1}, sb[4] = {1, 1, 1, 1}, x[256] = {}, s[4] = {};
  double out[4] = {};
  int64_t bad_row[1] = {2}, neg_col[1] = {-1};
  check(dgo_gemm_ref(nullptr, b, sa, sb, 1, 1, 64, 64, nullptr, 0, nullptr, 0, out, 1) == -1, "null a");
  check(dgo_gemm_ref(a, b, sa, sb, 1, 1, 96, 64, nullptr, 0, nullptr, 0, out, 1) == -1, "K % g");
  check(dgo_gemm_ref(a, b, sa, sb, 1, 1, 64, 0, nullptr, 0, nullptr, 0, out, 1) == -1, "g = 0");
  check(dgo_gemm_ref(a, b, sa, sb, 2, 1, 64, 64, bad_row, 1, nullptr, 0, out, 1) == -1, "row out of range");
  check(dgo_gemm_ref_fmt(a, b, sa, sb, 1, 1, 64, 64, 2, 0, nullptr, 0, nullptr, 0, out, 1) == -1, "bad format");
  check(dgo_gemm_ref_rowa(a, b, sa, sb, 1, 1, 64, 64, 0, 0, nullptr, 0, neg_col, 1, out, 1) == -1, "negative column");
  check(dgo_gemm_ref_layout(a, b, sa, sb, 1, 1, 64, 64, 4, 0, 0, nullptr, 0, nullptr, 0, out, 1) == -1, "bad layout");
  check(dgo_quantize_blocks(x, 1, 96, 64, q, s, 1) == -1, "cols % g");
  check(dgo_quantize_blocks_fmt(x, 1, 64, 64, 3, q, s, 1) == -1, "quantiser format");
  check(dgo_quantize_rows_fmt(x, 0, 64, 64, 0, q, s, 1) == -1, "zero rows");
  check(dgo_epilogue(out, 1, 1, nullptr, nullptr, 3) == -1, "bad activation");
}

}  // namespace

int main() {
  check(dgo_hardware_threads() >= 1, "hardware threads");
  codecs();
  quantisers(1, 64, 64, 1, 1);
  quantisers(130, 192, 64, 3, 2);
  quantisers(7, 256, 128, 4, 3);
  quantisers(300, 512, 256, 8, 4);
  gemms(1, 1, 64, 64, 1, 10);
  gemms(17, 15, 192, 64, 3, 11);
  gemms(65, 127, 384, 128, 4, 12);
  gemms(129, 33, 512, 256, 2, 13);
  gemms(200, 136, 256, 128, 16, 14);
  rejects();
  if (g_failures) {
    std::fprintf(stderr, "%d checks failed\n", g_failures);
    return 1;
  }
  std::printf("oracle checks passed\n");
  return 0;
}
