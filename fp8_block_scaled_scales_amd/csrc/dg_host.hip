// Host side of the C ABI declared in include/dg.h: argument checks, the
// one-time per-device architecture check, tile-table selection and launch.
//
// Tile selection replaces a runtime JIT with a small precompiled table
// (the pages describe compiling per shape at first use, DeepGEMM实战 §2.1, and
// precompiling common shapes, the DeepGEMM-style template article §2.3/§5.3;
// this library only does the latter).

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>

#include "../../include/dg.h"
#include "gemm_fp8_nt.h"
#include "quant_fp8.h"

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_status[kMaxDevices];  // DG_OK or DG_EUNSUPPORTED, set once per device

// Split-K plans (dg_gemm_fp8_ws only) are capped at this many FP32 partial
// floats, which bounds the workspace a caller provides.
constexpr int64_t kWsFloats = 4ll << 20;  // 16 MB of partial tiles

// When a workspace plan splits K. A split costs about 2 us beyond the
// streaming kernel's time for the same K range (the FP32 partials' trip
// through memory and the second kernel), and its 64x64 tiles move fewer
// bytes per CU only when there are few of them, so it pays where it cuts a
// long K range several times: at least kSplitMinSteps 128-byte K steps and
// at least kSplitMin splits (at most 32 tiles of 64x64, whatever M). Graph-timed
// on small M (8, 64, 128 rows, N 256 to 4096, g = 128, K 1024 to 32768):
// K >= 16384 with 8 to 16 splits took 0.46 to 0.81 of the streaming time,
// and with M 192 to 2048 (N 64 to 640, K 16384 to 65536, g 64 and 128) 0.46
// to 0.90 of the planned entry's; K = 7168 with 8 to 14 splits 0.91 to
// 1.15; K <= 4096 1.05 to 1.6; 4 splits 0.95 to 1.57 at any K; 2 splits
// (M = 128, N = 4096, whose streaming tiles take two rounds) 0.87 to 1.10.
// kMaxSplit bounds the second kernel's sum per output.
constexpr int64_t kSplitMinSteps = 128;
constexpr int64_t kSplitMin = 8;
constexpr int64_t kMaxSplit = 16;

// Workspace layout of a split-K plan: the FP32 partial tiles,
// [tile][split][bm][bn], row-major inside a tile.

// The workspace of dg_gemm_fp8_noalloc, for callers that cannot allocate
// device memory: a fixed array in the library's code object, one copy per GPU
// the library runs on, held until the process ends. Its host-side name is a
// stand-in, not a device address: the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is passed to kernels. A split-K call writes every partial it
// reads, so the array's contents never matter.
constexpr int64_t kScratchBytes = 4ll << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

void find_scratch(int dev) {
  void* p = nullptr;
  g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
}

thread_local hipError_t t_last_hip = hipSuccess;
thread_local char t_msg[256];

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("DG_LOG");
    return e && e[0] == '1';
  }();
  return on;
}

void check_device(int dev) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    g_dev_status[dev] = DG_EUNSUPPORTED;
    return;
  }
  g_dev_status[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? DG_OK : DG_EUNSUPPORTED;
}

// Argument checks shared by the GEMM and the tile query. No HIP call.
int validate(int64_t M, int64_t N, int64_t K, int gran) {
  if (M <= 0 || N <= 0 || K <= 0) return DG_EINVAL;
  if (M > DG_MAX_DIM || N > DG_MAX_DIM || K > DG_MAX_DIM) return DG_EINVAL;
  if (gran != 64 && gran != 128 && gran != 256) return DG_EINVAL;
  if (K % gran != 0) return DG_EINVAL;
  return DG_OK;
}

// K segment the kernels contract before each promotion: g itself for 64 and
// 128; g = 256 runs the 128 kernels with one scale factor per two segments.
int kernel_gran(int gran) { return gran > 128 ? 128 : gran; }

const dg::KernelEntry* find(int cls, int gran) {
  for (int i = 0; i < dg::kTableSize; ++i)
    if (dg::kTable[i].gran == gran && dg::kTable[i].cls == cls) return &dg::kTable[i];
  return nullptr;
}

struct Plan {
  const dg::KernelEntry* e;
  int ksplit;
  int64_t tiles;
};

// Tile-table choice (pure host arithmetic, no HIP call).
// Every shape takes the table entry of the call's granularity with the least
// estimated time (estimate_us), the whole K per workgroup: the 32x32
// streaming tiles (whose waves split K inside the workgroup), 64x64,
// 128x128, or the 256-row tiles 128 or 256 wide. With a workspace, a long K
// (kSplitMinSteps) that gives at least kSplitMin splits instead splits the
// K range of each 64x64 tile over several workgroups, until about
// one workgroup per CU (256) runs, at most kMaxSplit per tile and at least 4
// pipeline steps per split.
// DG_FORCE_TILE=<kernel id>, read at every call, replaces the choice when
// that entry has the call's granularity (tuning, benchmarking and tests; a
// split-K entry then runs with one split unless the call has a workspace).
int forced_tile() {
  const char* e = std::getenv("DG_FORCE_TILE");
  return e ? std::atoi(e) : -1;
}

int64_t splits_for(const dg::KernelEntry* e, int64_t tiles, int64_t nsteps) {
  int64_t ks = (256 + tiles / 2) / tiles;
  ks = std::min<int64_t>(std::min<int64_t>(ks, kMaxSplit), nsteps / 4);
  while (ks > 1 && tiles * ks * e->bm * e->bn > kWsFloats) --ks;
  return std::max<int64_t>(ks, 1);
}

int64_t tiles_of(const dg::KernelEntry* e, int64_t M, int64_t N) {
  return ((M + e->bm - 1) / e->bm) * ((N + e->bn - 1) / e->bn);
}

// Estimated microseconds of one launch of e on M x N x K (whole K per
// workgroup). Every class is held back by how fast one CU pulls its tile's
// operand rows from L2 (the workgroups of one CU share that rate) or by its
// arithmetic, so a launch takes the entry's fixed cost plus, per round of
// one tile per CU, a fixed cost and the larger of moving bm + bn rows of K
// bytes and 2 bm bn K FLOP at the entry's per-CU rates. The constants were
// fitted by least squares in log time to graph-timed launches of every
// entry on 166 shapes (M 32 to 4096, N 1024 to 28672, K 2048 to 8192,
// g 64 and 128); the least estimate picked an entry within 3% of the
// fastest on every one of them.
double estimate_us(const dg::KernelEntry* e, int64_t M, int64_t N, int64_t K) {
  const int64_t rounds = (tiles_of(e, M, N) + 255) / 256;
  const double bytes = (double)(e->bm + e->bn) * (double)K;
  const double flop = 2.0 * e->bm * e->bn * (double)K;
  return e->launch_us +
         (double)rounds * (e->round_us + std::max(bytes / (e->cu_gbps * 1e3), flop / (e->cu_tflops * 1e6)));
}

Plan plan(int64_t M, int64_t N, int64_t K, int sgran, bool split_ok) {
  Plan p{nullptr, 1, 0};
  const int gran = kernel_gran(sgran);
  const int64_t nsteps = (K + 127) / 128;
  auto split_k = [&]() {
    p.e = find(dg::kClassSplitK, gran);
    p.tiles = tiles_of(p.e, M, N);
    p.ksplit = split_ok ? (int)splits_for(p.e, p.tiles, nsteps) : 1;
    return p;
  };
  const int force = forced_tile();
  if (force >= 0) {
    for (int i = 0; i < dg::kTableSize; ++i)
      if (dg::kTable[i].id == force && dg::kTable[i].gran == gran) p.e = &dg::kTable[i];
    if (p.e) {
      p.tiles = tiles_of(p.e, M, N);
      if (p.e->cls == dg::kClassSplitK && split_ok) p.ksplit = (int)splits_for(p.e, p.tiles, nsteps);
      return p;
    }
  }
  if (split_ok && nsteps >= kSplitMinSteps && split_k().ksplit >= kSplitMin) return p;
  // The entry with the least estimated time: small tiles where there are few
  // of them (fewer bytes per CU, more CUs busy), large ones where the
  // arithmetic dominates.
  p = Plan{nullptr, 1, 0};
  double best = 0.0;
  for (int i = 0; i < dg::kTableSize; ++i) {
    const dg::KernelEntry* e = &dg::kTable[i];
    if (e->gran != gran) continue;
    const double t = estimate_us(e, M, N, K);
    if (!p.e || t < best) {
      best = t;
      p.e = e;
    }
  }
  p.tiles = tiles_of(p.e, M, N);
  p.ksplit = 1;
  return p;
}

// Workspace bytes of a plan: none without a K split.
int64_t workspace_bytes(const Plan& p) {
  if (p.ksplit <= 1) return 0;
  return p.tiles * p.ksplit * p.e->bm * p.e->bn * (int64_t)sizeof(float);
}

// One-time per-device check; returns DG_OK, DG_EUNSUPPORTED or DG_ELAUNCH.
int device_ready(int* dev_out = nullptr) {
  int dev = 0;
  if ((t_last_hip = hipGetDevice(&dev)) != hipSuccess) return DG_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return DG_EUNSUPPORTED;
  std::call_once(g_dev_once[dev], check_device, dev);
  if (dev_out) *dev_out = dev;
  return g_dev_status[dev];
}

}  // namespace

namespace {

// Layout check shared by the GEMM and the tile query: a known code. A
// transposed operand's stored rows (M bytes for A [K,M], N for B [K,N]) may
// have any length: its tiles are copied in 16-byte pieces along those rows
// whatever their alignment, and the bytes a piece takes past a row's end
// belong to rows of A or B past M or N, whose outputs are never stored.
int validate_layout(int64_t M, int64_t N, int layout) {
  (void)M;
  (void)N;
  if (layout < DG_LAYOUT_NT || layout > DG_LAYOUT_TN) return DG_EINVAL;
  return DG_OK;
}

// Whether the byte ranges [p, p + n) and [q, q + m) share a byte (empty
// ranges share none).
bool overlaps(const void* p, uint64_t n, const void* q, uint64_t m) {
  const uintptr_t x = (uintptr_t)p, y = (uintptr_t)q;
  return n && m && x < y + m && y < x + n;
}

// split_ok: few-tile long-K shapes may split K over workgroups, through ws (the
// caller's, ws_bytes long; none when ws_bytes is 0) or, with use_scratch,
// through the library's static scratch array.
int gemm(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M, int64_t N, int64_t K,
         int gran, int layout, int sa_rows, int fmt_a, int fmt_b, const float* bias, int act, void* stream,
         bool split_ok = false, void* ws = nullptr, int64_t ws_bytes = 0, bool use_scratch = false) {
  if (!a || !b || !sa || !sb || !out) return DG_EINVAL;
  if (sa_rows != gran && sa_rows != 1) return DG_EINVAL;
  if (validate_layout(M, N, layout) != DG_OK) return DG_EINVAL;
  if ((fmt_a != DG_FMT_E4M3 && fmt_a != DG_FMT_E5M2) || (fmt_b != DG_FMT_E4M3 && fmt_b != DG_FMT_E5M2))
    return DG_EINVAL;
  if (act != DG_ACT_NONE && act != DG_ACT_RELU && act != DG_ACT_GELU) return DG_EINVAL;
  if ((uintptr_t)bias & 3) return DG_EALIGN;
  if (ws_bytes < 0 || (ws_bytes > 0 && !ws) || (ws && ws_bytes == 0)) return DG_EINVAL;
  if ((uintptr_t)ws & 255) return DG_EALIGN;
  int rc = validate(M, N, K, gran);
  if (rc != DG_OK) return rc;
  if (((uintptr_t)a & 15) || ((uintptr_t)b & 15) || ((uintptr_t)sa & 3) || ((uintptr_t)sb & 3) ||
      ((uintptr_t)out & 1))
    return DG_EALIGN;
  // A workspace lets few-tile long-K shapes split K; without one nothing does.
  Plan pl = plan(M, N, K, gran, split_ok && (ws_bytes > 0 || use_scratch));
  if (!pl.e || pl.tiles * pl.ksplit > 0x7fffffff) return DG_EINVAL;
  const int64_t need = workspace_bytes(pl);
  if (ws_bytes > 0 && ws_bytes < need) return DG_EINVAL;
  if (use_scratch && need > kScratchBytes) return DG_ESCRATCH;
  {
    // out is written while the inputs are read: it may overlap none of them
    // (the inputs may overlap each other), nor the workspace. Sizes are the
    // logical ones, which every layout stores in the same number of bytes.
    const uint64_t nks = (uint64_t)(K / gran);
    const uint64_t sa_rows_n = sa_rows == 1 ? (uint64_t)M : (uint64_t)((M + gran - 1) / gran);
    const uint64_t ob = 2ull * (uint64_t)M * (uint64_t)N;
    const uint64_t ab = (uint64_t)M * (uint64_t)K, bb = (uint64_t)N * (uint64_t)K;
    const uint64_t sab = 4ull * sa_rows_n * nks, sbb = 4ull * (uint64_t)((N + gran - 1) / gran) * nks;
    const uint64_t biasb = bias ? 4ull * (uint64_t)N : 0, wsb = (uint64_t)ws_bytes;
    if (overlaps(out, ob, a, ab) || overlaps(out, ob, b, bb) || overlaps(out, ob, sa, sab) ||
        overlaps(out, ob, sb, sbb) || overlaps(out, ob, bias, biasb))
      return DG_EINVAL;
    if (overlaps(ws, wsb, a, ab) || overlaps(ws, wsb, b, bb) || overlaps(ws, wsb, sa, sab) ||
        overlaps(ws, wsb, sb, sbb) || overlaps(ws, wsb, bias, biasb) || overlaps(ws, wsb, out, ob))
      return DG_EINVAL;
  }

  int dev = 0;
  rc = device_ready(&dev);
  if (rc != DG_OK) return rc;
  const dg::KernelEntry* e = pl.e;
  if (use_scratch && pl.ksplit > 1) {
    std::call_once(g_scratch_once[dev], find_scratch, dev);
    if (!g_scratch[dev]) {
      t_last_hip = g_scratch_err[dev];
      return DG_ELAUNCH;
    }
    ws = g_scratch[dev];
  }

  dg::GemmArgs p;
  p.a = static_cast<const uint8_t*>(a);
  p.b = static_cast<const uint8_t*>(b);
  p.sa = sa;
  p.sb = sb;
  p.out = static_cast<uint16_t*>(out);
  p.M = M;
  p.N = N;
  p.K = K;
  p.gran = kernel_gran(gran);
  p.sshift = gran == 256 ? 1 : 0;
  p.fmt = (fmt_a == DG_FMT_E5M2 ? 1 : 0) | (fmt_b == DG_FMT_E5M2 ? 2 : 0);
  p.rowa = sa_rows == 1 ? 1 : 0;
  p.layout = layout;
  p.vec_store = (((uintptr_t)out & 15) == 0 && N % 8 == 0) ? 1 : 0;
  p.ksplit = pl.ksplit;
  p.ws = pl.ksplit > 1 ? static_cast<float*>(ws) : nullptr;
  p.bias = bias;
  p.act = act;
  if (log_enabled())
    std::fprintf(stderr,
                 "dg_gemm_fp8 M=%lld N=%lld K=%lld g=%d layout=%d sa_rows=%d fmt=%d,%d bias=%d act=%d -> kernel %d "
                 "(%dx%d, %d stages, %d waves) ksplit %d grid %lld workspace %lld\n",
                 (long long)M, (long long)N, (long long)K, gran, layout, sa_rows, fmt_a, fmt_b, bias ? 1 : 0, act, e->id,
                 e->bm, e->bn, e->stages, e->waves, pl.ksplit, (long long)(pl.tiles * pl.ksplit), (long long)need);
  // the streaming entries take every layout themselves
  t_last_hip = layout == DG_LAYOUT_NT || e->cls == dg::kClassStream
                   ? e->launch(p, static_cast<hipStream_t>(stream))
                   : dg::launch_layout(e->id, p, static_cast<hipStream_t>(stream));
  return t_last_hip == hipSuccess ? DG_OK : DG_ELAUNCH;
}

// block_rows: rows per block, gran (g x g blocks) or 1 (1 x g blocks); in:
// DG_IN_F32, DG_IN_BF16 or DG_IN_F16.
int quantize(const void* x, int in, int64_t rows, int64_t cols, int gran, int block_rows, int fmt, void* q,
             float* scales, void* stream) {
  if (!x || !q || !scales) return DG_EINVAL;
  if (fmt != DG_FMT_E4M3 && fmt != DG_FMT_E5M2) return DG_EINVAL;
  if (in != DG_IN_F32 && in != DG_IN_BF16 && in != DG_IN_F16) return DG_EINVAL;
  const uint64_t esize = in == DG_IN_F32 ? 4 : 2;
  if (rows <= 0 || cols <= 0 || rows > DG_MAX_DIM || cols > DG_MAX_DIM) return DG_EINVAL;
  if ((gran != 64 && gran != 128 && gran != 256) || cols % gran != 0) return DG_EINVAL;
  if (block_rows != gran && block_rows != 1) return DG_EINVAL;
  if (((rows + block_rows - 1) / block_rows) * (cols / gran) > 0x7fffffff) return DG_EINVAL;
  // a lane writes one code per element of its 16-byte load: 4 bytes, or 8 for 16-bit input
  if (((uintptr_t)x & 15) || ((uintptr_t)q & (16 / esize - 1)) || ((uintptr_t)scales & 3)) return DG_EALIGN;
  {
    const uint64_t xb = esize * (uint64_t)rows * (uint64_t)cols, qb = (uint64_t)rows * (uint64_t)cols;
    const uint64_t sbytes = 4ull * (uint64_t)((rows + block_rows - 1) / block_rows) * (uint64_t)(cols / gran);
    if (overlaps(x, xb, q, qb) || overlaps(x, xb, scales, sbytes) || overlaps(q, qb, scales, sbytes)) return DG_EINVAL;
  }
  const int rc = device_ready();
  if (rc != DG_OK) return rc;
  dg::QuantArgs p;
  p.x = x;
  p.q = static_cast<uint8_t*>(q);
  p.scales = scales;
  p.rows = rows;
  p.cols = cols;
  p.gran = gran;
  p.fmt = fmt;
  p.in = in;
  if (log_enabled())
    std::fprintf(stderr, "dg_quantize_fp8 rows=%lld cols=%lld block %dx%d fmt=%d in=%d\n", (long long)rows,
                 (long long)cols, block_rows, gran, fmt, in);
  t_last_hip = block_rows == 1 ? dg::launch_quant_rows(p, static_cast<hipStream_t>(stream))
                               : dg::launch_quant(p, static_cast<hipStream_t>(stream));
  return t_last_hip == hipSuccess ? DG_OK : DG_ELAUNCH;
}

}  // namespace

extern "C" {

int dg_version(void) { return DG_VERSION; }

const char* dg_strerror(int code) {
  switch (code) {
    case DG_OK: return "success";
    case DG_EINVAL:
      return "invalid argument (null pointer, bad dimension, K not a multiple of gran, gran not 64/128/256, "
             "sa_rows neither gran nor 1, a format code other than DG_FMT_E4M3/DG_FMT_E5M2, an unknown "
             "activation or layout, an "
             "output or workspace that overlaps another argument, or a workspace smaller than the plan needs)";
    case DG_EALIGN:
      return "misaligned pointer (a, b need 16 bytes; sa, sb, bias 4 bytes; out 2 bytes; workspace 256 bytes)";
    case DG_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case DG_ESCRATCH:
      return "the call's K split needs more workspace than dg_gemm_fp8_noalloc's fixed scratch "
             "(dg_noalloc_scratch_bytes()); use dg_gemm_fp8_ws with a workspace of dg_query_tile_ws's size";
    case DG_ELAUNCH:
      std::snprintf(t_msg, sizeof t_msg, "HIP error %d: %s", (int)t_last_hip, hipGetErrorString(t_last_hip));
      return t_msg;
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

int query(int64_t M, int64_t N, int64_t K, int gran, int layout, bool split_ok, dg_tile_info* info) {
  if (!info) return DG_EINVAL;
  int rc = validate(M, N, K, gran);
  if (rc != DG_OK) return rc;
  if ((rc = validate_layout(M, N, layout)) != DG_OK) return rc;
  const Plan p = plan(M, N, K, gran, split_ok);
  if (!p.e || p.tiles * p.ksplit > 0x7fffffff) return DG_EINVAL;
  info->kernel_id = p.e->id;
  info->bm = p.e->bm;
  info->bn = p.e->bn;
  info->bk = 128;
  info->stages = p.e->stages;
  info->waves = p.e->waves;
  info->ksplit = p.ksplit;
  info->grid = p.tiles * p.ksplit;
  info->workspace_bytes = workspace_bytes(p);
  return DG_OK;
}

}  // namespace

extern "C" {

int dg_query_tile_layout(int64_t M, int64_t N, int64_t K, int gran, int layout, dg_tile_info* info) {
  return query(M, N, K, gran, layout, false, info);
}

int dg_query_tile_ws(int64_t M, int64_t N, int64_t K, int gran, int layout, dg_tile_info* info) {
  return query(M, N, K, gran, layout, true, info);
}

int dg_gemm_fp8_noalloc(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M,
                        int64_t N, int64_t K, int gran, int layout, int sa_rows, int fmt_a, int fmt_b,
                        const float* bias, int act, void* stream) {
  return gemm(a, b, sa, sb, out, M, N, K, gran, layout, sa_rows, fmt_a, fmt_b, bias, act, stream, true, nullptr, 0,
              true);
}

int64_t dg_noalloc_scratch_bytes(void) { return kScratchBytes; }

int dg_query_tile(int64_t M, int64_t N, int64_t K, int gran, dg_tile_info* info) {
  return dg_query_tile_layout(M, N, K, gran, DG_LAYOUT_NT, info);
}

int dg_gemm_fp8_ws(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M, int64_t N,
                   int64_t K, int gran, int layout, int sa_rows, int fmt_a, int fmt_b, const float* bias, int act,
                   void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm(a, b, sa, sb, out, M, N, K, gran, layout, sa_rows, fmt_a, fmt_b, bias, act, stream, true, workspace,
              workspace_bytes);
}

int dg_gemm_fp8_nt(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M,
                   int64_t N, int64_t K, int gran, void* stream) {
  return gemm(a, b, sa, sb, out, M, N, K, gran, DG_LAYOUT_NT, gran, DG_FMT_E4M3, DG_FMT_E4M3, nullptr, DG_ACT_NONE,
              stream);
}

int dg_gemm_fp8_nt_fmt(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M,
                       int64_t N, int64_t K, int gran, int fmt_a, int fmt_b, void* stream) {
  return gemm(a, b, sa, sb, out, M, N, K, gran, DG_LAYOUT_NT, gran, fmt_a, fmt_b, nullptr, DG_ACT_NONE, stream);
}

int dg_gemm_fp8_nt_epi(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M,
                       int64_t N, int64_t K, int gran, int fmt_a, int fmt_b, const float* bias, int act,
                       void* stream) {
  return gemm(a, b, sa, sb, out, M, N, K, gran, DG_LAYOUT_NT, gran, fmt_a, fmt_b, bias, act, stream);
}

int dg_gemm_fp8_nt_ex(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M,
                      int64_t N, int64_t K, int gran, int sa_rows, int fmt_a, int fmt_b, const float* bias, int act,
                      void* stream) {
  return gemm(a, b, sa, sb, out, M, N, K, gran, DG_LAYOUT_NT, sa_rows, fmt_a, fmt_b, bias, act, stream);
}

int dg_gemm_fp8_layout(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M,
                       int64_t N, int64_t K, int gran, int layout, int fmt_a, int fmt_b, const float* bias, int act,
                       void* stream) {
  return gemm(a, b, sa, sb, out, M, N, K, gran, layout, gran, fmt_a, fmt_b, bias, act, stream);
}

int dg_quantize_fp8_blocks(const float* x, int64_t rows, int64_t cols, int gran, int fmt, void* q, float* scales,
                           void* stream) {
  return quantize(x, DG_IN_F32, rows, cols, gran, gran, fmt, q, scales, stream);
}

int dg_quantize_fp8_rows(const float* x, int64_t rows, int64_t cols, int gran, int fmt, void* q, float* scales,
                         void* stream) {
  return quantize(x, DG_IN_F32, rows, cols, gran, 1, fmt, q, scales, stream);
}

int dg_quantize_e4m3_blocks(const float* x, int64_t rows, int64_t cols, int gran, void* q, float* scales,
                            void* stream) {
  return quantize(x, DG_IN_F32, rows, cols, gran, gran, DG_FMT_E4M3, q, scales, stream);
}

int dg_quantize_fp8_blocks_typed(const void* x, int in_type, int64_t rows, int64_t cols, int gran, int fmt, void* q,
                                 float* scales, void* stream) {
  return quantize(x, in_type, rows, cols, gran, gran, fmt, q, scales, stream);
}

int dg_quantize_fp8_rows_typed(const void* x, int in_type, int64_t rows, int64_t cols, int gran, int fmt, void* q,
                               float* scales, void* stream) {
  return quantize(x, in_type, rows, cols, gran, 1, fmt, q, scales, stream);
}

}  // extern "C"
