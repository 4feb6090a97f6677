// Device helpers shared by the gfx950 GEMM kernels: vector types, the
// explicit memory-counter wait, the XCD-aware tile order, raw buffer
// descriptors and the HBM->LDS copy of a staged slab.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

// vmcnt(n) with expcnt and lgkmcnt left at their maxima (gfx9 encoding).
#define DG_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8))

// Race check build (compiled with -DDG_EXTRA_SYNC into libdg_sync.so): every
// pipeline step ends with all of the wave's memory operations drained (every
// copy in flight landed, every LDS read done) and, in the kernels whose waves
// share the LDS ring, a workgroup barrier (the extra barrier per buffer switch
// of the template article, §5.5). The ring's own waits and barriers are meant
// to make these redundant, so this build must give the release build's bits:
// a difference means a slot was read before its copy landed or refilled
// while still being read. DG_STEP_SYNC_WAVE is for the per-wave rings, whose
// waves run different step counts and so cannot meet at extra barriers.
#ifdef DG_EXTRA_SYNC
#define DG_STEP_SYNC_WG()            \
  do {                               \
    __builtin_amdgcn_s_waitcnt(0);   \
    __syncthreads();                 \
  } while (0)
#define DG_STEP_SYNC_WAVE() __builtin_amdgcn_s_waitcnt(0)
#else
#define DG_STEP_SYNC_WG() \
  do {                    \
  } while (0)
#define DG_STEP_SYNC_WAVE() \
  do {                      \
  } while (0)
#endif

// Workgroup id -> (split, tile row, tile col).
// The dispatcher hands workgroup i to XCD i % 8. Renumber so that each XCD
// owns a contiguous run of the logical order. The logical order runs over the
// K splits slowest, then walks the tiles of one split as a grouped raster:
// GROUP_M tile rows advance together along N, so the tiles resident on one XCD
// share A row panels and B column panels of the same K range.
template <int GROUP_M>
__device__ __forceinline__ void map_tile(int tiles_m, int tiles_n, int& ks, int& tm, int& tn) {
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  const int xcd = pid & 7, local = pid >> 3, q = nwg >> 3, r = nwg & 7;
  pid = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
  const int tiles = tiles_m * tiles_n;
  ks = pid / tiles;
  pid -= ks * tiles;
  const int group = GROUP_M * tiles_n;
  const int gid = pid / group;
  const int first = gid * GROUP_M;
  const int gsz = min(tiles_m - first, GROUP_M);
  const int in = pid - gid * group;
  tm = first + in % gsz;
  tn = in / gsz;
}

// Buffer descriptor as four SGPRs: base, stride 0 (raw buffer), range in
// bytes, and the same config word as above.
__device__ __forceinline__ v4i rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return (v4i){(int)(uint32_t)p, (int)(uint32_t)(p >> 32) & 0xFFFF, (int)bytes, 0x00020000};
}

// One 16-byte-per-lane HBM->LDS copy: lane L's 16 bytes land at LDS byte
// lds_addr + 16*L. Written as inline assembly so that the compiler's wait
// insertion, which cannot tell the ring slots apart, does not wait for every
// slot before each LDS read; the kernel waits for these loads itself
// (wait_steps), in issue order, before the barrier that publishes a slot.
// The buffer offset is voff (per lane) + soff (wave-uniform).
__device__ __forceinline__ void lds_dma16(v4i rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff = 0) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}

// One 4-byte-per-lane HBM->LDS copy: lane L's 4 bytes land at LDS byte
// lds_addr + 4*L; otherwise as lds_dma16.
__device__ __forceinline__ void lds_dma4(v4i rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff = 0) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}

// Per-row A factors of one pipeline step (A scaled per row and K segment,
// 1 x g blocks): an FP32 array [SEGS][ROWS] in LDS, entry seg*ROWS + r the
// factor of tile row r for the step's K segment seg. Copied in 64-entry
// pieces; piece p (entries 64p .. 64p+63) lands at lds + 256*p, entries past
// ROWS*SEGS read zero into the padding. rsa covers the tile's rows of the
// [M][nks] factor tensor from the tile's first row (rows past M read zero);
// ks0 is the factor column of the step's first segment. valid = false moves
// no data (both offsets past any descriptor range, without wrapping).
template <int ROWS, int SEGS>
__device__ __forceinline__ void stage_row_scales(v4i rsa, uint8_t* lds, uint32_t nks, uint32_t ks0, int piece,
                                                 int lane, bool valid = true) {
  const uint32_t e = (uint32_t)(piece * 64 + lane);
  const uint32_t voff = e < (uint32_t)(ROWS * SEGS) ? ((e % ROWS) * nks + e / ROWS) * 4u : 0x40000000u;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  lds_dma4(rsa, __builtin_amdgcn_readfirstlane(lds_base + piece * 256), voff,
           __builtin_amdgcn_readfirstlane(valid ? ks0 * 4u : 0x40000000u));
}

// One instruction of a slab copy: rows 8*grp .. 8*grp+7 of a [rows x 128-byte]
// slab starting at column byte k0 of the rows the descriptor covers, into
// LDS at lds + 1024*grp (64 lanes x 16 B, written lane-contiguously from the
// wave-uniform LDS address). Lane L writes physical chunk L%8 of row L/8, so
// it fetches logical chunk (L%8) ^ key(row): the XOR swizzle is applied on
// the global-address side. SW = 0: key = row % 8, so 8 consecutive rows read
// at one logical chunk hit 8 distinct 16-byte bank groups of a 128-byte bank
// row; SW = 1: key = (row / 2) % 8, distinct 16-byte positions over 16
// consecutive rows of a 256-byte bank row; SW = 2: key = (row % 8) ^
// ((row / 8) % 2), which is both (conflict free whether a 16-byte read is
// served 8 lanes per clock over 128 bytes or 16 lanes over 256).
// The wave-uniform part of the offset (row group and K position) goes in the
// instruction's scalar offset, so a wave's copies share one or two per-lane
// offset registers.
//
// valid = false turns the copy into one that moves no data: the scalar offset
// is put past any descriptor range (offsets at or past the range read zero).
template <int SW>
__device__ __forceinline__ void stage_group(v4i rsrc, uint8_t* lds, uint32_t K, uint32_t k0, int grp, int lane,
                                            bool valid = true) {
  static_assert(SW >= 0 && SW <= 2, "swizzle");
  const uint32_t r_in = (uint32_t)lane >> 3;
  // key(row) with row = 8*grp + r_in
  const uint32_t key = SW == 0   ? r_in
                       : SW == 1 ? ((((uint32_t)grp & 1) << 2) + (r_in >> 1)) & 7
                                 : r_in ^ ((uint32_t)grp & 1);
  const uint32_t chunk = ((uint32_t)lane & 7) ^ key;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  lds_dma16(rsrc, __builtin_amdgcn_readfirstlane(lds_base + grp * 1024), r_in * K + chunk * 16,
            __builtin_amdgcn_readfirstlane(valid ? (uint32_t)grp * 8 * K + k0 : 0x80000000u));
}

// The whole slab of ROWS rows, split evenly over the workgroup's waves.
template <int ROWS, int NWAVES, int SW = 0>
__device__ __forceinline__ void stage_slab(v4i rsrc, uint8_t* lds, uint32_t K, uint32_t k0, int wave, int lane) {
  constexpr int GROUPS = ROWS / 8;
  static_assert(GROUPS % NWAVES == 0, "slab rows must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < GROUPS / NWAVES; ++i) stage_group<SW>(rsrc, lds, K, k0, i * NWAVES + wave, lane);
}

// Transposed operands (DeepGEMM实战 §3.3: A stored [K,M] or B stored [K,N]).
// A step's tile of such an operand is staged as its 128 K rows of W bytes
// (the tile's M or N extent: 64, 128 or 256), 16-byte chunks XOR-swizzled by
// row, and read into the MFMA fragment with the transposing LDS read.
//
// Swizzle key of row r. A transposing read is served 32 lanes (256 bytes,
// all 64 banks) per clock: two 16-lane groups, each eight consecutive rows
// at one or two adjacent logical chunks, and the two groups either 32 rows
// apart at the same chunk (16x16 fragment) or at the same rows one chunk apart
// (32x32 fragment). The key spreads all of that over distinct banks:
//   256-byte rows (one row = all banks): 2*(r%8) puts the eight rows on even
//     chunk offsets, and bit 0 flips every 32 rows, so the neighbouring chunk
//     or the group 32 rows on lands on the odd ones;
//   128-byte rows (two rows = all banks): r%8 already separates the eight
//     rows (odd rows sit in the other half of the banks), and bit 0 flips
//     every 32 rows;
//   64-byte rows (four rows = all banks): rows four apart share bank offsets,
//     so bit 1 flips with (r/4)%2 and bit 0 every 32 rows.
//   32-byte rows (the streaming class): the eight rows a 32-lane half reads
//     are 256 contiguous bytes already, so no swizzle.
template <int W>
__device__ __forceinline__ int tkey(int row) {
  static_assert(W == 32 || W == 64 || W == 128 || W == 256, "transposed tile width");
  const int far = (row >> 5) & 1;
  return W == 32    ? 0
         : W == 64  ? ((((row >> 2) & 1) << 1) | far)
         : W == 128 ? ((row & 7) ^ far)
                    : ((2 * (row & 7)) ^ far);
}

// One instruction of a transposed tile's copy: rows RPI*grp .. RPI*grp+RPI-1
// (RPI = 1024/W) of the step's K rows, all W bytes, into LDS at
// lds + 1024*grp. Lane L writes physical chunk L % (W/16) of its row, so it
// fetches the logical chunk that belongs there. rsrc's base is the step's first
// K row at the tile's first column; pitch is the stored row length (M or N).
template <int W>
__device__ __forceinline__ void stage_group_t(v4i rsrc, uint8_t* lds, uint32_t pitch, int grp, int lane) {
  constexpr int CPR = W / 16, RPI = 64 / CPR;
  const int r_in = lane / CPR, p = lane % CPR;
  const uint32_t c = (uint32_t)(p ^ tkey<W>(grp * RPI + r_in));
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  lds_dma16(rsrc, __builtin_amdgcn_readfirstlane(lds_base + grp * 1024), (uint32_t)r_in * pitch + c * 16,
            __builtin_amdgcn_readfirstlane((uint32_t)grp * RPI * pitch));
}

// Byte range of the descriptor a transposed tile's step copies read through:
// the step's K rows (k0 .. k0 + rows - 1) of a stored [K, len] operand from
// column col0 on. A 16-byte piece of the tile's last column chunk may reach
// past a stored row's end when len is not a multiple of 16; the range check
// drops a 4-byte word that reaches past the range whole, so the range runs 16
// bytes into the next K row when there is one (past the last row see
// patch_tail_t).
__device__ __forceinline__ uint32_t tile_range_t(int64_t k0, int K, int len, int col0, int BKr) {
  const int64_t rows = min((int64_t)BKr, (int64_t)K - k0);
  return (uint32_t)(rows * len - col0 + (k0 + rows < K ? 16 : 0));
}

// The tensor's last step has no row after it to run into. There the range
// check drops the 4-byte words that reach past the tensor's end, and every
// byte such a word holds lies in the tensor's last 3 bytes (a dropped word
// starts less than 4 bytes before the end). With rows of 4 bytes or more
// those are the last len % 4 bytes of the last K row; with rows of 1 to 3
// bytes they reach back over up to 3 rows. Lanes 0-2 each take one of the
// last 3 bytes (global offset total - 1 - lane, total = K * len) and, when it
// lies in this step's rows (from k0) and the W-wide tile from col0, write it
// from memory into the slab at its swizzled place. Writing a byte that was
// not dropped writes the value already there. src is the tensor's base.
// Called between two barriers: after every wave's copies of the step have
// landed, before any wave reads the slab (or, for a wave's private ring, after
// that wave's own copies have landed).
template <int W>
__device__ __forceinline__ void patch_tail_t(uint8_t* slab, const uint8_t* src, int64_t total, int len, int64_t k0,
                                             int col0, int lane) {
  const int64_t e = total - 1 - lane;
  if (lane < 3 && e >= 0) {
    const int64_t row = e / len;
    const int col = (int)(e - row * len);
    if (row >= k0 && col >= col0 && col < col0 + W) {
      const int r = (int)(row - k0), t = col - col0;
      slab[r * W + (((t >> 4) ^ tkey<W>(r)) << 4) + (t & 15)] = src[e];
    }
  }
}

// The 32 K bytes of this lane's 32x32x64 fragment from a transposed tile:
// lane l needs column col0 + l%32 (its row of A, or of B) at K bytes
// kofs + 32*(l/32) .. +31. ds_read_b64_tr_b8 works on 16-lane groups: lane
// 16G + 8h + j receives byte j of the eight 8-byte rows addressed by lanes
// 16G + h, 16G + 2 + h, ..., 16G + 14 + h, in that order (measured on gfx950
// with an address-coded LDS pattern). So lane x addresses row
// kofs + 32*(x/32) + 8q + (x%16)/2 at column col0 + 16*((x/16)%2) + 8*(x%2),
// and read q = 0..3 brings K bytes 8q .. 8q+7 of the lane's own column.
template <int W>
__device__ __forceinline__ v8i frag_tr(const uint8_t* slab, int col0, int kofs, int lane) {
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
  const int row0 = kofs + 32 * (lane >> 5) + ((lane & 15) >> 1);
  v2i r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = row0 + 8 * q;
    const int off = row * W + (((col >> 4) ^ tkey<W>(row)) << 4) + (col & 15);
    r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(lds_void_t*)(const_cast<uint8_t*>(slab) + off));
  }
  return (v8i){r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
}

// The same for the 16x16x128 fragment: lane l needs column col0 + l%16 at K
// bytes kofs + 32*(l/16) .. +31. With the 16-lane groups above, group G is
// K quarter G and half-group h columns 8h .. 8h+7, so lane x addresses row
// kofs + 32*(x/16) + 8q + (x%16)/2 at column col0 + 8*(x%2).
template <int W>
__device__ __forceinline__ v8i frag_tr16(const uint8_t* slab, int col0, int kofs, int lane) {
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  const int col = col0 + 8 * (lane & 1);
  const int row0 = kofs + 32 * (lane >> 4) + ((lane & 15) >> 1);
  v2i r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = row0 + 8 * q;
    const int off = row * W + (((col >> 4) ^ tkey<W>(row)) << 4) + (col & 15);
    r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(lds_void_t*)(const_cast<uint8_t*>(slab) + off));
  }
  return (v8i){r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
}

// Epilogue before the BF16 store (the template article's extension point
// before the write-back, §2.3 and §6: bias add, ReLU, GELU), in FP32:
// y = act(x + b) with b = bias[column] when a bias is given, act none, ReLU,
// or GELU in its exact form 0.5 * y * (1 + erf(y / sqrt 2)). EPI selects the
// compiled form: 0 = no bias and no activation (x passes unchanged, and the
// kernel holds no epilogue state at all), 1 = optional bias and optional
// ReLU, 2 = optional bias and GELU. It is a template parameter because the
// epilogue is unrolled over every accumulator register: a runtime choice
// would leave an inlined erf behind a branch at each of them, code the
// instruction cache would fetch around per element.
// erf by the rational approximation of Abramowitz and Stegun, Handbook of
// Mathematical Functions, formula 7.1.26: for z >= 0,
// erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2) with
// t = 1 / (1 + p z), absolute error below 1.5e-7; odd in z. Straight-line
// (one reciprocal, one exponential, a few FMAs): the epilogue inlines it once
// per accumulator register.
__device__ __forceinline__ float erf_as7126(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, az, 1.0f));
  float poly = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  poly = __builtin_fmaf(poly, t, 1.421413741f);
  poly = __builtin_fmaf(poly, t, -0.284496736f);
  poly = __builtin_fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f(-az * az * 1.4426950408889634f);  // exp(-z^2)
  return copysignf(1.0f - poly * e, z);
}

template <int EPI>
__device__ __forceinline__ float epilogue_fn(float x, bool has_bias, float b, bool relu) {
  if constexpr (EPI == 0) return x;
  if (has_bias) x += b;
  if constexpr (EPI == 1) {
    if (relu) x = fmaxf(x, 0.0f);
  }
  if constexpr (EPI == 2) x = 0.5f * x * (1.0f + erf_as7126(x * 0.70710678118654752f));
  return x;
}

// Compiled epilogue form of a call (see epilogue_fn): 0 without bias and
// activation, 2 for GELU, 1 otherwise.
inline int epilogue_form(const float* bias, int act) { return act == 2 ? 2 : (bias || act == 1) ? 1 : 0; }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // v_cvt_pk_bf16_f32: nearest even
}

}  // namespace dg
