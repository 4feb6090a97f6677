// The library's host-side logic (argument checks, tile plans, workspace
// sizes, status texts) under AddressSanitizer and UndefinedBehaviorSanitizer,
// built by tests/test_sanitize.py for the CPU only: the library's sources are
// compiled without device code and linked into this program, which needs no
// GPU. Every GEMM and quantiser call below carries one argument error, so
// each returns before its first HIP call and no kernel is ever launched (the
// pointers are plain addresses the host code never dereferences); the tile
// queries are pure host arithmetic over a grid of shapes up to the largest
// accepted sizes and past them. Exit status 0 when every call returns what
// the header promises.

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dg.h"

namespace {

int g_failures = 0;

void expect(int got, int want, const char* what, long long a = 0, long long b = 0) {
  if (got != want) {
    ++g_failures;
    std::fprintf(stderr, "FAILED: %s (%lld, %lld): got %d, want %d\n", what, a, b, got, want);
  }
}

// Distinct, well-aligned fake device addresses, far apart.
void* addr(int i) { return reinterpret_cast<void*>((uintptr_t)(i + 1) << 40); }
const float* faddr(int i) { return static_cast<const float*>(addr(i)); }
void* shift(void* p, uintptr_t by) { return reinterpret_cast<void*>(reinterpret_cast<uintptr_t>(p) + by); }

void tiles() {
  const int64_t dims[] = {-1, 0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 4096, 8192,
                          DG_MAX_DIM - 1, DG_MAX_DIM, DG_MAX_DIM + 1, (int64_t)1 << 31, (int64_t)1 << 40};
  const int64_t ks[] = {-128, 0, 64, 128, 192, 256, 7168, 16384, DG_MAX_DIM, DG_MAX_DIM + 256};
  const int grans[] = {0, 32, 64, 128, 256, 512};
  for (int64_t M : dims)
    for (int64_t N : dims)
      for (int64_t K : ks)
        for (int g : grans)
          for (int layout = -1; layout <= 4; ++layout) {
            dg_tile_info t, tw;
            std::memset(&t, 0xAB, sizeof t);
            const int rc = dg_query_tile_layout(M, N, K, g, layout, &t);
            const int rcw = dg_query_tile_ws(M, N, K, g, layout, &tw);
            if (rc != rcw) expect(rcw, rc, "ws query agrees on validity", M, N);
            const bool valid = M >= 1 && N >= 1 && K >= 1 && M <= DG_MAX_DIM && N <= DG_MAX_DIM &&
                               K <= DG_MAX_DIM && (g == 64 || g == 128 || g == 256) && K % g == 0 && layout >= 0 &&
                               layout <= 3;
            // valid sizes are refused only when the grid would pass 2^31 - 1
            // workgroups (M x N beyond 2^31 tiles of at least 32 x 32)
            const bool huge = (double)M * (double)N >= 1e12;
            if (!(valid && huge && rc == DG_EINVAL)) expect(rc, valid ? DG_OK : DG_EINVAL, "query validity", M, N);
            if (rc != DG_OK) continue;
            const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
            expect(t.ksplit, 1, "no K split without a workspace", M, N);
            expect(t.workspace_bytes == 0, 1, "no workspace without one", M, N);
            expect(t.grid == tiles, 1, "grid = tiles", M, N);
            expect(t.bk, 128, "bk", M, N);
            const int64_t twt = ((M + tw.bm - 1) / tw.bm) * ((N + tw.bn - 1) / tw.bn);
            expect(tw.grid == twt * tw.ksplit, 1, "ws grid = tiles x ksplit", M, N);
            expect((tw.ksplit > 1) == (tw.workspace_bytes > 0), 1, "workspace iff split", M, N);
            if (layout == 0) {
              dg_tile_info n;
              expect(dg_query_tile(M, N, K, g, &n), DG_OK, "NT query", M, N);
              expect(n.kernel_id == t.kernel_id && n.bm == t.bm && n.bn == t.bn && n.bk == t.bk &&
                         n.stages == t.stages && n.waves == t.waves && n.ksplit == t.ksplit && n.grid == t.grid &&
                         n.workspace_bytes == t.workspace_bytes,
                     1, "NT query = layout 0 query", M, N);
            }
          }
  expect(dg_query_tile(64, 64, 128, 128, nullptr), DG_EINVAL, "null info");
  expect(dg_query_tile_ws(64, 64, 128, 128, 0, nullptr), DG_EINVAL, "null info (ws)");
}

// One GEMM call with a single defect; every one of them must be refused.
void gemm_rejects() {
  void *a = addr(0), *b = addr(1), *out = addr(4), *ws = addr(6);
  const float *sa = faddr(2), *sb = faddr(3), *bias = faddr(5);
  const int64_t M = 64, N = 4096, K = 7168;
  expect(dg_gemm_fp8_nt(nullptr, b, sa, sb, out, M, N, K, 128, nullptr), DG_EINVAL, "null a");
  expect(dg_gemm_fp8_nt(a, nullptr, sa, sb, out, M, N, K, 128, nullptr), DG_EINVAL, "null b");
  expect(dg_gemm_fp8_nt(a, b, nullptr, sb, out, M, N, K, 128, nullptr), DG_EINVAL, "null sa");
  expect(dg_gemm_fp8_nt(a, b, sa, nullptr, out, M, N, K, 128, nullptr), DG_EINVAL, "null sb");
  expect(dg_gemm_fp8_nt(a, b, sa, sb, nullptr, M, N, K, 128, nullptr), DG_EINVAL, "null out");
  expect(dg_gemm_fp8_nt(a, b, sa, sb, out, 0, N, K, 128, nullptr), DG_EINVAL, "M = 0");
  expect(dg_gemm_fp8_nt(a, b, sa, sb, out, M, -5, K, 128, nullptr), DG_EINVAL, "N < 0");
  expect(dg_gemm_fp8_nt(a, b, sa, sb, out, M, N, K + 64, 128, nullptr), DG_EINVAL, "K % g");
  expect(dg_gemm_fp8_nt(a, b, sa, sb, out, M, N, K, 96, nullptr), DG_EINVAL, "gran 96");
  expect(dg_gemm_fp8_nt(a, b, sa, sb, out, DG_MAX_DIM + 1, N, K, 128, nullptr), DG_EINVAL, "M too large");
  expect(dg_gemm_fp8_nt(shift(a, 8), b, sa, sb, out, M, N, K, 128, nullptr), DG_EALIGN, "a misaligned");
  expect(dg_gemm_fp8_nt(a, shift(b, 4), sa, sb, out, M, N, K, 128, nullptr), DG_EALIGN, "b misaligned");
  expect(dg_gemm_fp8_nt(a, b, (const float*)shift((void*)sa, 2), sb, out, M, N, K, 128, nullptr), DG_EALIGN,
         "sa misaligned");
  expect(dg_gemm_fp8_nt(a, b, sa, sb, shift(out, 1), M, N, K, 128, nullptr), DG_EALIGN, "out misaligned");
  // out overlapping an input (the first byte of A's last row)
  expect(dg_gemm_fp8_nt(a, b, sa, sb, shift(a, (M - 1) * K), M, N, K, 128, nullptr), DG_EINVAL, "out overlaps a");
  expect(dg_gemm_fp8_nt(a, b, sa, sb, shift((void*)sb, 4), M, N, K, 128, nullptr), DG_EINVAL, "out overlaps sb");
  expect(dg_gemm_fp8_nt_fmt(a, b, sa, sb, out, M, N, K, 128, 2, 0, nullptr), DG_EINVAL, "fmt_a 2");
  expect(dg_gemm_fp8_nt_fmt(a, b, sa, sb, out, M, N, K, 128, 0, -1, nullptr), DG_EINVAL, "fmt_b -1");
  expect(dg_gemm_fp8_nt_epi(a, b, sa, sb, out, M, N, K, 128, 0, 0, bias, 3, nullptr), DG_EINVAL, "act 3");
  expect(dg_gemm_fp8_nt_epi(a, b, sa, sb, out, M, N, K, 128, 0, 0, (const float*)shift((void*)bias, 2), 1, nullptr),
         DG_EALIGN, "bias misaligned");
  expect(dg_gemm_fp8_nt_epi(a, b, sa, sb, out, M, N, K, 128, 0, 0, (const float*)out, 1, nullptr), DG_EINVAL,
         "bias overlaps out");
  expect(dg_gemm_fp8_nt_ex(a, b, sa, sb, out, M, N, K, 128, 64, 0, 0, nullptr, 0, nullptr), DG_EINVAL,
         "sa_rows 64 with g 128");
  expect(dg_gemm_fp8_layout(a, b, sa, sb, out, M, N, K, 128, 4, 0, 0, nullptr, 0, nullptr), DG_EINVAL, "layout 4");
  expect(dg_gemm_fp8_layout(a, b, sa, sb, out, M, N, K, 128, -1, 0, 0, nullptr, 0, nullptr), DG_EINVAL,
         "layout -1");
  // the workspace call: size, alignment, presence and overlap rules
  dg_tile_info t;
  expect(dg_query_tile_ws(64, 512, 32768, 128, 0, &t), DG_OK, "ws plan");
  const int64_t need = t.workspace_bytes;
  expect(need > 0, 1, "a split plan needs a workspace");
  expect(dg_gemm_fp8_ws(a, b, sa, sb, out, 64, 512, 32768, 128, 0, 128, 0, 0, nullptr, 0, ws, need - 1, nullptr),
         DG_EINVAL, "workspace too small");
  expect(dg_gemm_fp8_ws(a, b, sa, sb, out, 64, 512, 32768, 128, 0, 128, 0, 0, nullptr, 0, shift(ws, 128), need,
                        nullptr),
         DG_EALIGN, "workspace misaligned");
  expect(dg_gemm_fp8_ws(a, b, sa, sb, out, 64, 512, 32768, 128, 0, 128, 0, 0, nullptr, 0, nullptr, need, nullptr),
         DG_EINVAL, "size without a workspace");
  expect(dg_gemm_fp8_ws(a, b, sa, sb, out, 64, 512, 32768, 128, 0, 128, 0, 0, nullptr, 0, ws, -1, nullptr), DG_EINVAL,
         "negative workspace size");
  expect(dg_gemm_fp8_ws(a, b, sa, sb, out, 64, 512, 32768, 128, 0, 128, 0, 0, nullptr, 0, ws, 0, nullptr), DG_EINVAL,
         "workspace without a size");
  expect(dg_gemm_fp8_ws(a, b, sa, sb, out, 64, 512, 32768, 128, 0, 128, 0, 0, nullptr, 0, out, need, nullptr),
         DG_EINVAL, "workspace overlaps out");
  expect(dg_gemm_fp8_ws(a, b, sa, sb, out, 64, 512, 32768, 128, 0, 128, 0, 0, nullptr, 0, shift(a, 256), need,
                        nullptr),
         DG_EINVAL, "workspace overlaps a");
  expect(dg_gemm_fp8_noalloc(a, b, sa, sb, out, 64, 512, 32768, 96, 0, 96, 0, 0, nullptr, 0, nullptr), DG_EINVAL,
         "noalloc gran 96");
  expect(dg_gemm_fp8_noalloc(a, b, sa, sb, shift(out, 1), 64, 512, 32768, 128, 0, 128, 0, 0, nullptr, 0, nullptr),
         DG_EALIGN, "noalloc out misaligned");
}

void quant_rejects() {
  const float* x = faddr(0);
  void* q = addr(1);
  float* s = const_cast<float*>(faddr(2));
  expect(dg_quantize_e4m3_blocks(nullptr, 64, 128, 128, q, s, nullptr), DG_EINVAL, "null x");
  expect(dg_quantize_e4m3_blocks(x, 0, 128, 128, q, s, nullptr), DG_EINVAL, "rows 0");
  expect(dg_quantize_e4m3_blocks(x, 64, 192, 128, q, s, nullptr), DG_EINVAL, "cols % g");
  expect(dg_quantize_fp8_blocks(x, 64, 128, 128, 2, q, s, nullptr), DG_EINVAL, "fmt 2");
  expect(dg_quantize_fp8_rows(x, DG_MAX_DIM + 1, 128, 128, 0, q, s, nullptr), DG_EINVAL, "rows too large");
  expect(dg_quantize_fp8_rows(x, 64, 128, 128, 0, shift(q, 2), s, nullptr), DG_EALIGN, "q misaligned");
  expect(dg_quantize_fp8_blocks((const float*)shift((void*)x, 4), 64, 128, 128, 0, q, s, nullptr), DG_EALIGN,
         "x misaligned");
  expect(dg_quantize_fp8_blocks(x, 64, 128, 128, 0, shift((void*)x, 64), s, nullptr), DG_EINVAL, "q overlaps x");
  // 2^31 or more scale factors
  expect(dg_quantize_fp8_rows(x, DG_MAX_DIM, DG_MAX_DIM - 128, 64, 0, q, s, nullptr), DG_EINVAL, "too many factors");
  // the typed calls: input kind, the 8-byte q alignment of 16-bit input, the
  // overlap rule on 2-byte elements
  expect(dg_quantize_fp8_blocks_typed(x, 3, 64, 128, 128, 0, q, s, nullptr), DG_EINVAL, "typed kind 3");
  expect(dg_quantize_fp8_rows_typed(x, -1, 64, 128, 128, 0, q, s, nullptr), DG_EINVAL, "typed kind -1");
  expect(dg_quantize_fp8_rows_typed(x, DG_IN_BF16, 64, 128, 128, 0, shift(q, 4), s, nullptr), DG_EALIGN,
         "typed bf16 q misaligned");
  expect(dg_quantize_fp8_blocks_typed(shift((void*)x, 8), DG_IN_F16, 64, 128, 128, 0, q, s, nullptr), DG_EALIGN,
         "typed f16 x misaligned");
  expect(dg_quantize_fp8_blocks_typed(x, DG_IN_BF16, 64, 128, 128, 0, shift((void*)x, 8192), s, nullptr),
         DG_EINVAL, "typed q overlaps bf16 x");
  expect(dg_quantize_fp8_blocks_typed(x, DG_IN_BF16, 64, 192, 128, 0, q, s, nullptr), DG_EINVAL, "typed cols % g");
}

void status_texts() {
  expect(dg_version(), DG_VERSION, "version");
  expect(dg_noalloc_scratch_bytes() > 0, 1, "scratch size");
  for (int code = -16; code <= 16; ++code) {
    if (code == DG_ELAUNCH) continue;  // asks the HIP runtime for its last error's text
    const char* s = dg_strerror(code);
    expect(s != nullptr && std::strlen(s) > 0, 1, "status text", code);
  }
}

}  // namespace

int main() {
  tiles();
  gemm_rejects();
  quant_rejects();
  status_texts();
  if (g_failures) {
    std::fprintf(stderr, "%d checks failed\n", g_failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
