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
#include <cstring>
#include <mutex>

#include "../../include/dg.h"
#include "gemm_fp8_nt.h"
#include "quant_e4m3.h"

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_status[kMaxDevices];  // DG_OK or DG_EUNSUPPORTED, set once per device

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
  if (gran != 64 && gran != 128) return DG_EINVAL;
  if (K % gran != 0) return DG_EINVAL;
  return DG_OK;
}

const dg::KernelEntry* select(int64_t M, int64_t N, int64_t K, int gran) {
  (void)M;
  (void)N;
  (void)K;
  for (int i = 0; i < dg::kTableSize; ++i)
    if (dg::kTable[i].gran == gran) return &dg::kTable[i];
  return nullptr;
}

// One-time per-device check; returns DG_OK, DG_EUNSUPPORTED or DG_ELAUNCH.
int device_ready() {
  int dev = 0;
  if ((t_last_hip = hipGetDevice(&dev)) != hipSuccess) return DG_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return DG_EUNSUPPORTED;
  std::call_once(g_dev_once[dev], check_device, dev);
  return g_dev_status[dev];
}

int64_t grid_of(const dg::KernelEntry* e, int64_t M, int64_t N) {
  return ((M + e->bm - 1) / e->bm) * ((N + e->bn - 1) / e->bn);
}

}  // namespace

extern "C" {

int dg_version(void) { return DG_VERSION; }

const char* dg_strerror(int code) {
  switch (code) {
    case DG_OK: return "success";
    case DG_EINVAL: return "invalid argument (null pointer, bad dimension, K not a multiple of gran, or gran not 64/128)";
    case DG_EALIGN: return "misaligned pointer (a, b need 16 bytes; sa, sb 4 bytes; out 2 bytes)";
    case DG_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case DG_ELAUNCH:
      std::snprintf(t_msg, sizeof t_msg, "HIP error %d: %s", (int)t_last_hip, hipGetErrorString(t_last_hip));
      return t_msg;
    default: return "unknown status";
  }
}

int dg_query_tile(int64_t M, int64_t N, int64_t K, int gran, dg_tile_info* info) {
  if (!info) return DG_EINVAL;
  const int rc = validate(M, N, K, gran);
  if (rc != DG_OK) return rc;
  const dg::KernelEntry* e = select(M, N, K, gran);
  if (!e || grid_of(e, M, N) > 0x7fffffff) return DG_EINVAL;
  info->kernel_id = e->id;
  info->bm = e->bm;
  info->bn = e->bn;
  info->bk = 128;
  info->stages = e->stages;
  info->waves = e->waves;
  info->ksplit = e->ksplit;
  info->grid = grid_of(e, M, N);
  return DG_OK;
}

int dg_gemm_fp8_nt(const void* a, const void* b, const float* sa, const float* sb, void* out, int64_t M,
                   int64_t N, int64_t K, int gran, void* stream) {
  if (!a || !b || !sa || !sb || !out) return DG_EINVAL;
  int rc = validate(M, N, K, gran);
  if (rc != DG_OK) return rc;
  if (((uintptr_t)a & 15) || ((uintptr_t)b & 15) || ((uintptr_t)sa & 3) || ((uintptr_t)sb & 3) ||
      ((uintptr_t)out & 1))
    return DG_EALIGN;
  const dg::KernelEntry* e = select(M, N, K, gran);
  if (!e || grid_of(e, M, N) > 0x7fffffff) return DG_EINVAL;

  rc = device_ready();
  if (rc != DG_OK) return rc;

  dg::GemmArgs p;
  p.a = static_cast<const uint8_t*>(a);
  p.b = static_cast<const uint8_t*>(b);
  p.sa = sa;
  p.sb = sb;
  p.out = static_cast<uint16_t*>(out);
  p.M = M;
  p.N = N;
  p.K = K;
  p.gran = gran;
  p.vec_store = (((uintptr_t)out & 15) == 0 && N % 8 == 0) ? 1 : 0;
  if (log_enabled())
    std::fprintf(stderr, "dg_gemm_fp8_nt M=%lld N=%lld K=%lld g=%d -> kernel %d (%dx%d, %d stages, %d waves) grid %lld\n",
                 (long long)M, (long long)N, (long long)K, gran, e->id, e->bm, e->bn, e->stages, e->waves,
                 (long long)grid_of(e, M, N));
  t_last_hip = e->launch(p, static_cast<hipStream_t>(stream));
  return t_last_hip == hipSuccess ? DG_OK : DG_ELAUNCH;
}

int dg_quantize_e4m3_blocks(const float* x, int64_t rows, int64_t cols, int gran, void* q, float* scales,
                            void* stream) {
  if (!x || !q || !scales) return DG_EINVAL;
  if (rows <= 0 || cols <= 0 || rows > DG_MAX_DIM || cols > DG_MAX_DIM) return DG_EINVAL;
  if ((gran != 64 && gran != 128) || cols % gran != 0) return DG_EINVAL;
  if (((rows + gran - 1) / gran) * (cols / gran) > 0x7fffffff) return DG_EINVAL;
  if (((uintptr_t)x & 15) || ((uintptr_t)q & 3) || ((uintptr_t)scales & 3)) return DG_EALIGN;
  const int rc = device_ready();
  if (rc != DG_OK) return rc;
  dg::QuantArgs p;
  p.x = x;
  p.q = static_cast<uint8_t*>(q);
  p.scales = scales;
  p.rows = rows;
  p.cols = cols;
  p.gran = gran;
  if (log_enabled())
    std::fprintf(stderr, "dg_quantize_e4m3_blocks rows=%lld cols=%lld g=%d\n", (long long)rows, (long long)cols, gran);
  t_last_hip = dg::launch_quant_e4m3(p, static_cast<hipStream_t>(stream));
  return t_last_hip == hipSuccess ? DG_OK : DG_ELAUNCH;
}

}  // extern "C"
