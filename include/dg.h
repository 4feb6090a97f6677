/*
 * dg.h - C ABI of the block-scaled FP8 GEMM library for AMD MI355X (gfx950).
 *
 * The operation (DeepGEMM in practice / DeepGEMM实战: §2.2 one FP32 scale
 * factor per 128x128 block of each input, restored while the products are
 * accumulated; §3.2 FP32 accumulation, each K segment summed on its own and
 * the segments then added; §3.3 and §4.2 the NT layout, A [M,K] and B [N,K]
 * in FP8, preallocated BF16 output):
 *
 *   out[i,j] = bf16( sum_kb  sa[i/g, kb] * sb[j/g, kb] * P[i,j,kb] )
 *   P[i,j,kb] = sum_{k = kb*g}^{kb*g+g-1} A[i,k] * B[j,k]
 *
 * with A, B decoded from OCP E4M3FN codes, P accumulated in FP32 over exactly
 * one g-wide K segment, the promotion acc = fma(P, sa*sb, acc) done in FP32
 * once per segment, and the FP32 result rounded to BF16 (nearest even).
 * Summation order inside a segment is unspecified; results are deterministic
 * for a given (M, N, K, g) and device.
 *
 * All pointers are device pointers (memory the caller allocated, e.g. PyTorch
 * tensors). The library keeps no caller pointer after a call returns,
 * allocates no device memory at all, and the GEMM calls below need no
 * workspace: every K reduction of the default tile choice, small M included,
 * happens inside one workgroup. dg_gemm_fp8_ws is the one call that splits K
 * over several workgroups, through a workspace the caller passes in. Calls
 * are asynchronous on `stream` (a hipStream_t; NULL is the default stream);
 * faults during execution surface at the caller's next synchronisation. No
 * call prints unless the environment sets DG_LOG=1, and no call exits or
 * throws. DG_FORCE_TILE=<kernel id> in the environment, read at every call,
 * replaces the tile choice with that table entry where it has the call's
 * granularity (tuning and tests; results stay within the same tolerance,
 * with other bits).
 *
 * Thread safety: calls may come from several host threads and run
 * concurrently on any streams (dg_gemm_fp8_ws: each concurrent call with its
 * own workspace). The one-time per-device check (the architecture must be
 * gfx950) runs under std::call_once.
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. The split follows the pitfalls article (GPU GEMM history and
 * pitfalls, §5.4), which separates failures a caller can recover from (an
 * argument to fix and retry) from those it cannot (a failed launch or a
 * device fault, after which the caller should stop using the device): the
 * first three are the former, reported before any HIP call with nothing
 * launched; DG_ELAUNCH is the latter, with the HIP error kept for
 * dg_strerror. */
#define DG_OK 0
#define DG_EINVAL (-1)       /* bad argument; nothing was launched (recoverable) */
#define DG_EALIGN (-2)       /* misaligned pointer; nothing was launched (recoverable) */
#define DG_EUNSUPPORTED (-3) /* device is not gfx950; nothing was launched */
#define DG_ELAUNCH (-4)      /* a HIP call failed (not recoverable); dg_strerror() gives its text */
#define DG_ESCRATCH (-5)     /* dg_gemm_fp8_noalloc: the plan needs more than its fixed scratch; nothing launched */

/* Version of this header and library: 2.1.0 (2.0.0: dg_tile_info gained
 * workspace_bytes; dg_gemm_fp8_ws and dg_query_tile_ws were added; no call
 * but dg_gemm_fp8_ws splits K over workgroups. 2.1.0: the quantisers take
 * BF16 and FP16 input through the _typed calls). */
#define DG_VERSION 210

/* Largest accepted dimension, 2^24 - 256: a 256-row tile of K bytes per row
 * (256 * K) then stays below 2^32 bytes, the reach of a buffer descriptor,
 * so every in-tile byte offset fits 32 bits; a multiple of 256, so it is a
 * valid K for every g. */
#define DG_MAX_DIM ((1LL << 24) - 256)

/*
 * dg_gemm_fp8_nt - C[M,N] = A[M,K] * B[N,K]^T with g x g block scales.
 *
 *   a    E4M3FN codes, [M,K] row-major (K contiguous, lda = K). 16-byte aligned.
 *   b    E4M3FN codes, [N,K] row-major (K contiguous, ldb = K). 16-byte aligned.
 *   sa   FP32 scales of A, [ceil(M/g)][K/g] row-major. 4-byte aligned.
 *   sb   FP32 scales of B, [ceil(N/g)][K/g] row-major. 4-byte aligned.
 *   out  BF16 result, [M,N] row-major (ldc = N), fully overwritten. 2-byte
 *        aligned; must not overlap a, b, sa or sb (DG_EINVAL if it does;
 *        the inputs may overlap each other, e.g. a == b for A*A^T).
 *   M, N, K  > 0 and <= DG_MAX_DIM; K a multiple of gran.
 *   gran block granularity g: 64, 128 or 256 (the pages' 64x64, 128x128 and
 *        256x256 choices, DeepGEMM实战 §3.1). For 256 the kernels promote
 *        every 128 K (each half of a 256 segment is accumulated in FP32 and
 *        added with the block's factor), so results match the one-segment
 *        definition up to FP32 rounding, inside the stated tolerance.
 *   stream hipStream_t to enqueue on (NULL = default stream).
 *
 * Rows of A beyond M and rows of B beyond N are never read, and nothing
 * outside out[0..M-1][0..N-1] is written (ragged M and N are supported).
 * Returns DG_OK, DG_EINVAL (null pointer, bad dims, K % g != 0, bad g),
 * DG_EALIGN, DG_EUNSUPPORTED (not gfx950) or DG_ELAUNCH. Argument errors are
 * reported before any HIP call.
 */
int dg_gemm_fp8_nt(const void* a, const void* b, const float* sa, const float* sb, void* out,
                   int64_t M, int64_t N, int64_t K, int gran, void* stream);

/* FP8 formats of the operands (DeepGEMM实战 §2.2 names both as the inputs).
 * E5M2 is the OCP format torch.float8_e5m2 implements: bias 15, subnormals
 * m/4 * 2^-14, largest finite 57344, exponent field 31 = inf/NaN. */
#define DG_FMT_E4M3 0
#define DG_FMT_E5M2 1

/* Element types of the quantisers' input (dg_quantize_fp8_*_typed). */
#define DG_IN_F32 0
#define DG_IN_BF16 1
#define DG_IN_F16 2

/*
 * dg_gemm_fp8_nt_fmt - dg_gemm_fp8_nt with each operand's format given:
 * fmt_a, fmt_b each DG_FMT_E4M3 or DG_FMT_E5M2 (any of the four pairs).
 * Everything else, including layouts, scales, gran and status codes, is as
 * for dg_gemm_fp8_nt; (DG_FMT_E4M3, DG_FMT_E4M3) is that call. Codes that
 * decode to infinity or NaN give unspecified results.
 */
int dg_gemm_fp8_nt_fmt(const void* a, const void* b, const float* sa, const float* sb, void* out,
                       int64_t M, int64_t N, int64_t K, int gran, int fmt_a, int fmt_b, void* stream);

/* Epilogue activations (the template article's epilogue extension point,
 * §2.3 and §6: bias add, ReLU, GELU before the write-back). */
#define DG_ACT_NONE 0
#define DG_ACT_RELU 1
#define DG_ACT_GELU 2 /* exact form: 0.5 * y * (1 + erf(y / sqrt 2)) */

/*
 * dg_gemm_fp8_nt_epi - dg_gemm_fp8_nt_fmt with an epilogue fused before the
 * BF16 store:  out[i,j] = bf16( act( C[i,j] + bias[j] ) )  with C the FP32
 * block-scaled product and everything in FP32.
 *
 *   bias  FP32 [N] device pointer, 4-byte aligned, or NULL for no bias; it
 *         must not overlap out (DG_EINVAL).
 *   act   DG_ACT_NONE, DG_ACT_RELU or DG_ACT_GELU.
 *
 * With bias NULL and DG_ACT_NONE this is dg_gemm_fp8_nt_fmt, bit for bit.
 * DG_EINVAL for an unknown act, DG_EALIGN for a misaligned bias; otherwise as
 * dg_gemm_fp8_nt_fmt.
 */
int dg_gemm_fp8_nt_epi(const void* a, const void* b, const float* sa, const float* sb, void* out,
                       int64_t M, int64_t N, int64_t K, int gran, int fmt_a, int fmt_b, const float* bias,
                       int act, void* stream);

/*
 * dg_gemm_fp8_nt_ex - dg_gemm_fp8_nt_epi with A's scale blocks chosen:
 * sa_rows is the number of A rows one factor covers, gran (g x g blocks, as
 * in every call above) or 1 (per-row factors, 1 x g blocks: the per-channel
 * factors of the DeepGEMM-style template article, §3.4). With sa_rows = 1:
 *
 *   out[i,j] = bf16( act( sum_kb  sa[i, kb] * sb[j/g, kb] * P[i,j,kb] + bias[j] ) )
 *
 *   sa   FP32 [M][K/gran] row-major, 4-byte aligned (one factor per row of A
 *        and K segment; for gran 256 one per row and 256-wide segment).
 *
 * B keeps its g x g blocks. Same tile choice as the other calls (the mode
 * changes no tile). With sa_rows = gran this is dg_gemm_fp8_nt_epi, bit for
 * bit; with sa_rows = 1 and every row's factors equal to its g-block's, the
 * result equals the block-scaled call's bit for bit. DG_EINVAL for sa_rows
 * other than gran or 1; otherwise as dg_gemm_fp8_nt_epi.
 */
int dg_gemm_fp8_nt_ex(const void* a, const void* b, const float* sa, const float* sb, void* out,
                      int64_t M, int64_t N, int64_t K, int gran, int sa_rows, int fmt_a, int fmt_b,
                      const float* bias, int act, void* stream);

/* Operand layouts (DeepGEMM实战 §3.3: each of A and B may be stored
 * transposed; the kernels read it that way, with no transposed copy in
 * memory). Named as C = op(A) op(B): first letter A, second B, with op(B) = B^T
 * for B stored [N,K]. Bit 1: A stored [K,M]; bit 0: B stored [K,N]. */
#define DG_LAYOUT_NT 0 /* A [M,K], B [N,K]: both K-contiguous (the other calls) */
#define DG_LAYOUT_NN 1 /* A [M,K], B [K,N] */
#define DG_LAYOUT_TT 2 /* A [K,M], B [N,K] */
#define DG_LAYOUT_TN 3 /* A [K,M], B [K,N] */

/*
 * dg_gemm_fp8_layout - dg_gemm_fp8_nt_epi with the operands stored in any of
 * the four layouts:
 *
 *   a    A[i,k] at a[i*K + k] (NT, NN: [M,K]) or at a[k*M + i] (TT, TN: [K,M]).
 *   b    B[j,k] at b[j*K + k] (NT, TT: [N,K]) or at b[k*N + j] (NN, TN: [K,N]).
 *   sa, sb  the logical block factors, as in dg_gemm_fp8_nt: sa
 *        [ceil(M/g)][K/g], sb [ceil(N/g)][K/g], whatever the layout (a
 *        quantiser run on a stored [K,M] matrix gives the transpose of sa).
 *   layout  DG_LAYOUT_NT, _NN, _TT or _TN.
 *
 * The result is the same product, out[i,j] as in dg_gemm_fp8_nt_epi, for any
 * M and N (a stored row of M or N bytes need not be a multiple of 16 long);
 * a and b 16-byte aligned as before. Every layout gives dg_gemm_fp8_nt_epi's
 * result bit for bit (the same K order inside every product).
 * dg_query_tile_layout names the tile a layout runs: the NT choice.
 * dg_gemm_fp8_ws (with no workspace) takes a layout together with per-row A
 * factors.
 */
int dg_gemm_fp8_layout(const void* a, const void* b, const float* sa, const float* sb, void* out,
                       int64_t M, int64_t N, int64_t K, int gran, int layout, int fmt_a, int fmt_b,
                       const float* bias, int act, void* stream);

/* The tile-table entry a call with these sizes would use. DeepGEMM实战 §6
 * advises keeping a record of which configuration ran for which shape; this
 * is that record, from the same host logic the calls use, so a caller can log
 * it next to its timings (DG_LOG=1 prints it per call). */
typedef struct dg_tile_info {
  int kernel_id; /* identifier of the precompiled table entry */
  int bm, bn;    /* workgroup output tile */
  int bk;        /* K bytes staged per pipeline step */
  int stages;    /* LDS ring depth */
  int waves;     /* waves per workgroup */
  int ksplit;    /* workgroups sharing one output tile, each over a K range (1 = none) */
  int64_t grid;  /* workgroups of the GEMM kernel (a K split adds a second, smaller launch) */
  int64_t workspace_bytes; /* workspace dg_gemm_fp8_ws needs for this plan (0: none) */
} dg_tile_info;

/*
 * dg_query_tile - fill *info with the tile-table entry dg_gemm_fp8_nt would
 * launch for (M, N, K, gran): the entry with the least estimated launch time
 * (fixed costs, then operand bytes per CU and FLOP per CU at each entry's
 * measured rates, per round of one tile per CU).
 * Pure host logic, no HIP call. Returns DG_OK or
 * DG_EINVAL for arguments dg_gemm_fp8_nt would reject. ksplit is always 1
 * and workspace_bytes 0: this call never splits K over workgroups.
 */
int dg_query_tile(int64_t M, int64_t N, int64_t K, int gran, dg_tile_info* info);

/* dg_query_tile for dg_gemm_fp8_layout: the entry a call with this layout
 * would use (DG_EINVAL for a layout or a transposed row length that call
 * would reject). */
int dg_query_tile_layout(int64_t M, int64_t N, int64_t K, int gran, int layout, dg_tile_info* info);

/*
 * dg_gemm_fp8_ws - the GEMM with a caller-owned workspace that lets
 * shapes with few output tiles and a long K split K over several workgroups.
 *
 * DeepGEMM实战 §3.2 accumulates K in segments that are summed separately and
 * then added; §5.3 names too little parallelism as what holds back small
 * shapes. With K >= 16384 (128 steps of 128) and few enough output tiles
 * (M x N up to 32 tiles of 64x64) that each gets at least 8 workgroups (at most 16, about
 * 256 in all), this call gives each tile ksplit workgroups, each over a
 * contiguous range of K segments, which write their FP32 partial tiles to the
 * workspace; a second kernel on the same stream adds each tile's partials in
 * split order (so the result does not depend on which split ran when),
 * applies the epilogue and writes the BF16 tile. The split costs about 2 us
 * of its own, which shorter K ranges do not win back against the default
 * plan's split of K inside the workgroup. Every other shape runs exactly what
 * dg_gemm_fp8_layout / dg_gemm_fp8_nt_ex runs, bit for bit, and leaves the
 * workspace untouched.
 *
 *   a, b, sa, sb, out, M, N, K, gran, layout, fmt_a, fmt_b, bias, act
 *        as dg_gemm_fp8_layout.
 *   sa_rows   gran or 1, as dg_gemm_fp8_nt_ex, with any layout: sa is
 *        [M][K/gran] with sa_rows = 1 whatever the storage of A's codes.
 *   workspace device memory of at least workspace_bytes bytes, 256-byte
 *        aligned, owned by the caller, or NULL with workspace_bytes 0 (then no
 *        shape splits K). It must not overlap any other argument. Its
 *        contents need no initialisation and are scratch between calls: a
 *        call writes every partial it reads, within the same call.
 *   workspace_bytes  size of workspace; must be 0 or at least the
 *        workspace_bytes dg_query_tile_ws reports for the shape (DG_EINVAL
 *        otherwise).
 *
 * Concurrency: two calls that may run at the same time (different streams,
 * or a graph replay beside an eager call) must use different workspaces;
 * calls on one stream may share one. The two kernels of a split call are
 * ordered by the stream (or by the graph's edge when captured); no workgroup
 * waits for another. Returns the status codes of dg_gemm_fp8_layout.
 */
int dg_gemm_fp8_ws(const void* a, const void* b, const float* sa, const float* sb, void* out,
                   int64_t M, int64_t N, int64_t K, int gran, int layout, int sa_rows, int fmt_a, int fmt_b,
                   const float* bias, int act, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * dg_gemm_fp8_noalloc - dg_gemm_fp8_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same plans and the same results, bit for bit,
 * with the workspace taken from a fixed array inside the library instead of
 * an argument. The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine).
 *
 * The array is dg_noalloc_scratch_bytes() bytes (4 MiB) of device memory per
 * GPU the library runs on, held until the process ends; its device address
 * is looked up on the first call on each device. A shape whose plan needs a
 * larger workspace (dg_query_tile_ws) is rejected with DG_ESCRATCH before
 * anything is launched. Every call on one GPU shares that GPU's array: calls
 * that may overlap in time on one GPU (different streams, graph replays
 * beside eager calls) race and must not be made; calls on one stream may
 * follow each other freely. Arguments and other status codes as
 * dg_gemm_fp8_ws.
 */
int dg_gemm_fp8_noalloc(const void* a, const void* b, const float* sa, const float* sb, void* out,
                        int64_t M, int64_t N, int64_t K, int gran, int layout, int sa_rows, int fmt_a, int fmt_b,
                        const float* bias, int act, void* stream);

/* Bytes of the fixed scratch array dg_gemm_fp8_noalloc uses on each GPU. */
int64_t dg_noalloc_scratch_bytes(void);

/* The plan dg_gemm_fp8_ws runs for these sizes, with the workspace it needs
 * (info->workspace_bytes; 0 when the plan does not split K). Pure host
 * logic; DG_EINVAL for arguments dg_gemm_fp8_ws would reject. */
int dg_query_tile_ws(int64_t M, int64_t N, int64_t K, int gran, int layout, dg_tile_info* info);

/*
 * dg_quantize_e4m3_blocks - block quantisation FP32 -> E4M3FN, the step that
 * produces the GEMM's operands (DeepGEMM实战 §4.4: quantisation sits outside
 * the GEMM, activations are quantised online, and the granularity must match
 * the GEMM's; §2.2: one factor per block maps it into FP8 range; §5.2:
 * quantise by dividing).
 *
 *   x       FP32 [rows][cols] row-major, 16-byte aligned.
 *   q       E4M3FN codes out, [rows][cols] row-major, 4-byte aligned.
 *   scales  FP32 out, [ceil(rows/gran)][cols/gran] row-major, 4-byte aligned.
 *   rows, cols > 0 and <= DG_MAX_DIM; cols a multiple of gran; gran 64, 128
 *   or 256; at most 2^31 - 1 scale factors (DG_EINVAL beyond). x, q and
 *   scales must not overlap one another (DG_EINVAL).
 *
 * Per gran x gran block (rows past the end make edge blocks partial):
 * amax = max |x| over present elements, scale = amax / 448 in FP32 (1.0
 * where that is zero: an all-zero block, or a block so small that the
 * quotient underflows, whose values then encode as zeros), q = E4M3(x /
 * scale) with the correctly rounded FP32 quotient and round-to-nearest-even.
 * Inputs must be finite. Same status codes and
 * asynchrony as dg_gemm_fp8_nt.
 */
int dg_quantize_e4m3_blocks(const float* x, int64_t rows, int64_t cols, int gran, void* q, float* scales,
                            void* stream);

/*
 * dg_quantize_fp8_blocks - dg_quantize_e4m3_blocks for either format: fmt
 * DG_FMT_E4M3 (scale = amax / 448) or DG_FMT_E5M2 (scale = amax / 57344,
 * codes E5M2 with round-to-nearest-even). Same arguments otherwise.
 */
int dg_quantize_fp8_blocks(const float* x, int64_t rows, int64_t cols, int gran, int fmt, void* q,
                           float* scales, void* stream);

/*
 * dg_quantize_fp8_rows - dg_quantize_fp8_blocks with 1 x gran blocks: one
 * factor per row and gran-wide column segment (the per-row A factors that
 * dg_gemm_fp8_nt_ex takes with sa_rows = 1).
 *
 *   scales  FP32 out, [rows][cols/gran] row-major, 4-byte aligned.
 *
 * Per segment: amax = max |x| over its gran elements, scale = amax / fmax
 * (448 or 57344) in FP32 (1.0 where that is zero, as above), codes as
 * dg_quantize_fp8_blocks. Same arguments and status codes otherwise.
 */
int dg_quantize_fp8_rows(const float* x, int64_t rows, int64_t cols, int gran, int fmt, void* q,
                         float* scales, void* stream);

/*
 * dg_quantize_fp8_blocks_typed, dg_quantize_fp8_rows_typed - the two
 * quantisers above on FP32, BF16 or FP16 input: the weights and activations
 * to quantise arrive in FP16 or BF16 (DeepGEMM实战 §4.4), and reading them as
 * they are moves half the bytes of an FP32 copy.
 *
 *   x        [rows][cols] row-major elements of kind in_type, 16-byte aligned:
 *            DG_IN_F32 (float), DG_IN_BF16 (bfloat16 bit patterns: the high
 *            half of an FP32 pattern) or DG_IN_F16 (IEEE binary16).
 *   in_type  DG_IN_F32, DG_IN_BF16 or DG_IN_F16; anything else is DG_EINVAL.
 *   q        codes out, [rows][cols] row-major; 4-byte aligned for FP32
 *            input, 8-byte aligned for 16-bit input (DG_EALIGN otherwise).
 *   scales   as dg_quantize_fp8_blocks (g x g) or dg_quantize_fp8_rows (1 x g).
 *
 * Each element is widened exactly to FP32 and the rule is then the FP32 one,
 * so a 16-bit matrix and its FP32 copy give identical codes and factors.
 * Inputs must be finite. Other arguments, status codes and asynchrony as
 * dg_quantize_fp8_blocks; with DG_IN_F32 each call is that call (blocks) or
 * dg_quantize_fp8_rows (rows).
 */
int dg_quantize_fp8_blocks_typed(const void* x, int in_type, int64_t rows, int64_t cols, int gran, int fmt, void* q,
                                 float* scales, void* stream);
int dg_quantize_fp8_rows_typed(const void* x, int in_type, int64_t rows, int64_t cols, int gran, int fmt, void* q,
                               float* scales, void* stream);

/* Text for a status code (for DG_ELAUNCH: the last HIP error on this
 * thread), so a caller can log which class of failure (the pitfalls article
 * §5.4: recoverable or not) it met. The string is static, or thread-local for
 * DG_ELAUNCH; it stays valid until this thread's next call. */
const char* dg_strerror(int code);

/* DG_VERSION of the loaded library, for the same per-run record as
 * dg_query_tile (DeepGEMM实战 §6: log which build and configuration ran). */
int dg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
