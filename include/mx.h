/*
 * mx.h -- C ABI of libmx, OCP-microscaling (MX) quantize-and-GEMM for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  BF16 tensors are packed into MX operands -- E2M1
 * (MXFP4), E2M3 (MXFP6) or E4M3 (MXFP8) element codes with one E8M0
 * exponent per block of 32 elements -- and packed operands are multiplied
 * with the gfx950 block-scaled matrix cores.  Sources (pages, by title):
 *   [P1] "feat(mxfp6): MXFP6 (E2M3) Flux linears, a fused MLP, and the MLPerf
 *        recipe" (Primus pull request 1064)
 *   [P3] "MXFP4 training for Flux models" (ROCm Primus technical guide)
 *   [P4] "MXFP8 cudnn-fe Swiglu fused Grouped MLP fwd/bwd and wgrad group
 *        gemm" (ao pull request 5)
 * Element and scale encodings follow the OCP Microscaling Formats (MX) v1.0
 * specification, which the pages name but do not spell out.
 *
 * Conventions for every entry point.
 *  - Pointers named as tensors are DEVICE pointers, owned by the caller, who
 *    also allocates every output and work buffer.  The library allocates no
 *    memory and keeps no state beyond a per-device property cache.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously on it; the call returns once enqueued.
 *  - bf16 tensors are row-major and dense.  Every device pointer must be
 *    16-byte aligned.
 *  - Packed operands ("rows x K", bits = 4, 6 or 8 per element) are stored
 *    K-group-major, the layout the GEMM reads: K is cut into groups of 128
 *    elements, and each group holds, row after row, the group's codes of
 *    every row.  Codes: [ceil(K/128)][rows][16*bits] bytes, the 128 codes
 *    of (row, group q) packed as below at byte (q * rows + row) * 16*bits
 *    (mx_codes_bytes bytes).  E8M0 scales, one byte per (row, 32-block b):
 *    [ceil(K/128)][rows][4], the four blocks of a group forming a dword,
 *    (row, b) at byte (b/4 * rows + row) * 4 + b % 4 (mx_scales_bytes
 *    bytes).  Pad bytes of a partial last group are 0.  A GEMM stage then
 *    reads the codes and the scales of a panel of rows as contiguous runs.
 *    As in [P4] (the grouped kernels' blocked E8M0 scale ABI), the
 *    quantizer writes the blocking the GEMM reads.  A ragged-K group of
 *    rows [k0, k1), k0 and k1 multiples of 128, is the run of K groups
 *    k0/128 .. k1/128 - 1.  Packing of the codes within a group, block by
 *    block (32 elements): E2M1 element 2j in the low nibble of byte j and
 *    2j+1 in the high nibble, 16 B per block; E4M3 one byte per element,
 *    32 B per block; E2M3 a little-endian 6-bit stream, element j at bits
 *    [6j, 6j+6) of the block's 24 B, of which the first 16 B lie at byte
 *    16b of the group and the last 8 B at byte 64 + 8(b ^ s) (block
 *    b = 0..3, s = bit 4 of the row), so that each matrix-core operand is one
 *    16-byte and one 8-byte read, both free of LDS bank conflicts.
 *    Every GEMM computes C = A . B^T on two such operands (the NT layout of
 *    [P3], Troubleshooting).
 *  - Return value: MX_OK, or an mx_status error.  Arguments are validated on
 *    the host before anything is enqueued; on error nothing is enqueued and
 *    no output is touched.  There is no fallback path: a call the kernels
 *    cannot serve fails with an error.
 *  - Deterministic: no atomics; repeated calls give bitwise-identical results.
 */
#ifndef MX_H
#define MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,           /* a required pointer is NULL */
  MX_ERR_SHAPE = 2,          /* a size is negative, zero where it may not be, or not the multiple required */
  MX_ERR_ALIGN = 3,          /* a device pointer is not 16-byte aligned */
  MX_ERR_FORMAT = 4,         /* unknown format / scale mode / prologue / epilogue / mode, or a combination not served */
  MX_ERR_OFFSETS = 5,        /* group offsets break their contract (checked only when asked to) */
  MX_ERR_INDEX_OVERFLOW = 6, /* a tensor exceeds 2^31 bytes (the kernels use 32-bit offsets) */
  MX_ERR_DEVICE = 7,         /* no current device, or the current device is not gfx950 */
  MX_ERR_LAUNCH = 8,         /* the HIP runtime reported an error when enqueuing */
  MX_ERR_SCRATCH = 9         /* the call needs more than the library's static scratch holds (mx_quantize_noalloc) */
} mx_status;

/* ---------------------------------------------------------------- enums */
typedef enum { MX_E2M1 = 1, MX_E2M3 = 2, MX_E4M3 = 3 } mx_fmt;

/* E8M0 exponent selection per block of 32 (amax = largest |value|):
 *  FLOOR: X = floor(log2 amax) - 2 (emax of E2M1/E2M3), for MXFP4/MXFP6;
 *  RCEIL: X = smallest integer with 448 * 2^X >= amax, for MXFP8 ([P4]:
 *         the E8M0 conversion rounds upward).
 * X is clamped to [-127, 127]; amax == 0 gives X = -127; a block holding a
 * NaN or Inf gets the NaN scale 0xFF and all-zero codes. */
typedef enum { MX_SCALE_FLOOR = 0, MX_SCALE_RCEIL = 1 } mx_scale_mode;

/* Elementwise prologue applied before packing ([P1] description: the packer
 * takes the activation epilogue as its prologue).  Each result is rounded to
 * bf16 before rotation / amax.  With logical output v [R][C]:
 *  IDENTITY: v = x                           x [R][C]
 *  GELU:     v = gelu_tanh(x)                x = h [R][C]
 *  DGELU:    v = da * gelu_tanh'(h)          x = da [R][C], aux = h [R][C]
 *  SWIGLU:   v = silu(g) * u                 x = H [R][2C] = [gate | up]
 *  DSWIGLU:  C = 2F, x = dz [R][F], aux = H [R][2F]:
 *            v[:, :F] = dz * u * s * (1 + g*(1-s)),  v[:, F:] = dz * g * s,
 *            s = 1/(1+exp(-g)) ([P4]: sigmoid formed as 1/(1+exp(-x))).
 * exp and the tanh form are this library's own binary32 contract (Cody-Waite
 * reduction + degree-7 polynomial), so results are reproducible to the bit. */
typedef enum {
  MX_PRO_IDENTITY = 0,
  MX_PRO_GELU_TANH = 1,
  MX_PRO_DGELU_TANH = 2,
  MX_PRO_SWIGLU = 3,
  MX_PRO_DSWIGLU = 4
} mx_prologue;

typedef enum { MX_BF16 = 0, MX_F32 = 1 } mx_dtype;

typedef enum { MX_GROUPED_RAGGED_M = 0, MX_GROUPED_RAGGED_K = 1 } mx_grouped_mode;

typedef enum { MX_EPI_NONE = 0, MX_EPI_SWIGLU = 1, MX_EPI_DSWIGLU = 2 } mx_epilogue;

/* One packed operand: codes [ceil(K/128)][rows][16*bits] + scales [ceil(K/128)][rows][4] bytes. */
typedef struct {
  void* codes;
  void* scales;
} mx_packed;

/* ---------------------------------------------------------------- quantize */
/*
 * mx_quantize -- pack a bf16 tensor into MX operands ([P1] Summary and
 * commit messages: scale, optional Hadamard rotation, cast and bit-pack in
 * one pass; [P4] first commit message: rowwise 1x32 and columnwise 32x1).
 *
 *  x, aux       bf16 inputs of the prologue (see mx_prologue); aux NULL
 *               unless DGELU or DSWIGLU.  Shapes per batch entry.
 *  batch        number of independent [R][C] problems stored back to back
 *               (e.g. the G experts' weights); every pointer below advances by
 *               one problem's size per batch entry.  >= 1.
 *  R, C         logical size of the quantized tensor v; multiples of 32,
 *               R = 0 or C = 0 enqueues nothing and returns MX_OK.
 *  fmt          MX_E2M1, MX_E2M3 or MX_E4M3.
 *  scale_mode   MX_SCALE_FLOOR or MX_SCALE_RCEIL.
 *  hadamard     1: rotate every 32-block by the normalised 32-point
 *               Walsh-Hadamard matrix (Sylvester order) before amax ([P1]
 *               description: the rotation is folded into the packer).
 *               Rotation order: radix-2 butterfly, strides 1,2,4,8,16, every
 *               add rounded to binary32, one multiply by fl32(1/sqrt 32).
 *               Only with MX_E2M3.
 *  row_codes, row_scales   rowwise (1x32 along dim 1) operand, [R] x K=C.
 *  col_codes, col_scales   columnwise (32x1 along dim 0) operand written
 *                          transposed, i.e. K-major [C] x K=R.
 *               Either pair may be NULL (both members of a pair alike), not
 *               both.
 *               The batch stride of a scale buffer is mx_scales_bytes(rows, K).
 *  colsum_partials  fp32 [R/32][C]: per-32-row-block column sums of v before
 *               rotation, rows in increasing order from +0 ([P1] commit
 *               messages: the bias gradient is finished from the packer's
 *               per-column partials).  NULL for none.
 *  colsum       fp32 [C]: sum of the partials in increasing block order
 *               (one extra small launch).  Requires colsum_partials.  NULL
 *               for none.
 * Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_FORMAT,
 * MX_ERR_INDEX_OVERFLOW, MX_ERR_DEVICE, MX_ERR_LAUNCH.
 */
int mx_quantize(const void* x, const void* aux, int64_t batch, int64_t R, int64_t C, int fmt,
                int scale_mode, int hadamard, int prologue, void* row_codes, void* row_scales,
                void* col_codes, void* col_scales, float* colsum_partials, float* colsum,
                void* stream);

/*
 * mx_quantize_noalloc -- mx_quantize for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  The column-sum partials, the one work buffer of
 * mx_quantize, live in a static device array of the library instead of a
 * caller buffer; the caller passes only inputs and outputs.  Arguments and
 * results are those of mx_quantize with colsum_partials taken away: colsum
 * (fp32 [batch][C], or NULL for none) is bitwise what mx_quantize returns.
 *
 * Limit: batch * (R/32) * C * 4 bytes of partials must fit the static array
 * of MX_NOALLOC_SCRATCH_BYTES (16 MiB: 4M partials, e.g. R = 8192 tokens at
 * C = 16384 columns); a larger call returns MX_ERR_SCRATCH and enqueues
 * nothing.  The array is allocated once per GPU when the library is loaded
 * and stays until the process ends.  The call itself never allocates: no
 * hipMalloc, hipFree or allocating library routine, on any path.
 *
 * Every call on one GPU uses that GPU's one array.  Each call writes every
 * partial it reads before reading it, in stream order, so nothing needs
 * clearing; but two calls whose work overlaps in time on one GPU (different
 * streams, or host threads) race on the array and give wrong column sums.
 * Order such calls on one stream, or use mx_quantize with separate buffers.
 * Errors: those of mx_quantize, plus MX_ERR_SCRATCH.
 */
#define MX_NOALLOC_SCRATCH_BYTES (16u << 20)
int mx_quantize_noalloc(const void* x, const void* aux, int64_t batch, int64_t R, int64_t C, int fmt,
                        int scale_mode, int hadamard, int prologue, void* row_codes, void* row_scales,
                        void* col_codes, void* col_scales, float* colsum, void* stream);

/*
 * mx_quantize_sr -- mx_quantize for MXFP4 gradient packs with stochastic
 * rounding of the elements ([P3] Overview, configuration table: SR of the
 * FP4 gradient quantization, an optional switch).  Format E2M1, FLOOR
 * scales, no rotation, identity prologue; arguments, layouts and errors as
 * mx_quantize with those fixed.
 *
 * The scales are those of mx_quantize.  For an element with v = x / 2^X:
 * |v| >= 6 saturates to 6; otherwise, with grid neighbours lo <= |v| < hi
 * and t = (|v| - lo) / (hi - lo), the magnitude is hi iff
 * (r >> 8) < floor(t * 2^24), else lo; the sign is kept.  r is word i % 4 of
 * Philox4x32-10 (Salmon et al., SC 2011) at counter (i/4 mod 2^32,
 * i/4 div 2^32, axis, 0) with key (seed mod 2^32, seed div 2^32), where i is
 * the element's index in its packed operand, i = (batch entry * rows +
 * operand row) * K + k, and axis is 0 for the rowwise operand and 1 for the
 * columnwise one.  The same seed gives the same bytes on every run.
 */
int mx_quantize_sr(const void* x, int64_t batch, int64_t R, int64_t C, void* row_codes, void* row_scales,
                   void* col_codes, void* col_scales, float* colsum_partials, float* colsum, uint64_t seed,
                   void* stream);

/*
 * mx_quantize_many -- several packs of one format, scale mode, rotation and
 * prologue in a single launch, with the results of n mx_quantize calls made
 * with each item's arguments.  For callers that pack several tensors at
 * once (a linear layer's activation, weight and output gradient before its
 * forward, data-gradient and weight-gradient GEMMs, [P1] description): one
 * launch keeps every compute unit busy where n small launches each leave
 * the GPU idle while they start and drain.
 *
 *  items        host array of n items; each item's fields have the meaning
 *               and rules of the mx_quantize arguments of the same names
 *               (row / col: {codes, scales}, either pair {NULL, NULL}).  The
 *               outputs of distinct items must not overlap.
 *  n            1 <= n <= MX_QUANTIZE_MANY_MAX.
 *  fmt, scale_mode, hadamard, prologue   as for mx_quantize, shared by all
 *               items.
 * Items with R = 0 or C = 0 are skipped.  The colsum of an item that asks
 * for one is finished by one extra small launch per such item.
 * Errors: MX_ERR_NULL (items NULL, or an item's pointers as for
 * mx_quantize), MX_ERR_SHAPE (n out of range, or an item's sizes), then as
 * mx_quantize for the first failing item; nothing is enqueued on an error.
 */
#define MX_QUANTIZE_MANY_MAX 8
typedef struct {
  const void* x;
  const void* aux;
  int64_t batch, R, C;
  mx_packed row, col;
  float* colsum_partials;
  float* colsum;
} mx_quantize_item;

int mx_quantize_many(const mx_quantize_item* items, int n, int fmt, int scale_mode, int hadamard, int prologue,
                     void* stream);

/* ---------------------------------------------------------------- GEMM */
/*
 * mx_gemm -- C[m][n] = sum_k A[m][k] * B[n][k] (+ bias[n]) on packed
 * operands of one format, accumulated in binary32 by the scaled matrix
 * cores.  The forward uses A = rows of X, B = rows of W; dgrad A = rows of
 * dY, B = columns of W; wgrad A = columns of dY, B = columns of X, so K is
 * the token count ([P1] description: M, N and K must be multiples of 256
 * because the backward GEMMs use K as an output dimension).
 *
 *  a_codes, a_scales   A, [M] x K.      b_codes, b_scales   B, [N] x K.
 *  M, N, K      multiples of 256; M = 0 or N = 0 enqueues nothing.
 *  fmt          element format of both operands.
 *  bias         optional [N] vector (NULL for none), dtype bias_dtype, added
 *               to the binary32 accumulator before the single rounding of
 *               the store ([P1] commit messages: the bias joins the GEMM's
 *               store epilogue and the result is rounded once).
 *  c            output [M][ldc] of dtype c_dtype (MX_BF16 rounds to nearest
 *               even; MX_F32 stores the accumulator).  ldc >= N, a multiple
 *               of 8.
 * Tiling: the output is cut into 256x256, 256x192, 192x256, 192x192 or
 * 256x128 tiles, whichever costs the fewest rounds x tile area with one tile
 * per compute unit, unless the tuned table (mx_gemm_plan) holds a measured
 * tiling without a K split for this device, format and shape
 * (mx_gemm_tiled takes the shape from the caller).
 * Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_FORMAT,
 * MX_ERR_INDEX_OVERFLOW, MX_ERR_DEVICE, MX_ERR_LAUNCH.
 */
int mx_gemm(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales,
            int64_t M, int64_t N, int64_t K, int fmt, const void* bias, int bias_dtype, void* c,
            int c_dtype, int64_t ldc, void* stream);

/*
 * mx_gemm_accumulate -- C[m][n] += sum_k A[m][k] * B[n][k] (+ bias[n]): the
 * weight gradient added into a caller-owned main_grad buffer in the GEMM's
 * own store epilogue, so no separate add pass reads and writes it again.
 * [P1] commit messages (the MXFP6 wgrad written straight into main_grad by
 * the GEMM): the page's GEMM stores with beta = 0, which overwrites, and so
 * needs one microbatch per optimizer step; mx_gemm into main_grad is that
 * store.  This call is beta = 1, for several microbatches per step.
 *
 * Arguments, tiling and errors are those of mx_gemm; c is read and written
 * (bf16 or binary32, dtype c_dtype).  Arithmetic per element: the binary32
 * accumulator plus the bias, plus the previous c converted exactly to
 * binary32, then one rounding to c_dtype (nearest even for bf16).  The
 * result is bitwise round(fl32(fl32(acc + bias) + c_old)) where
 * fl32(acc + bias) is what mx_gemm stores with c_dtype = MX_F32.
 */
int mx_gemm_accumulate(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales,
                       int64_t M, int64_t N, int64_t K, int fmt, const void* bias, int bias_dtype, void* c,
                       int c_dtype, int64_t ldc, void* stream);

/*
 * mx_gemm_tiled -- mx_gemm with the output tiling chosen by the caller:
 * tile_m x tile_n output tiles with wg_per_cu workgroups resident per
 * compute unit, one of
 *   256x256, 256x192, 192x256, 192x192, 256x128 at wg_per_cu = 1, and
 *   256x128, 128x256, 192x192 at wg_per_cu = 2 (each workgroup then takes at
 *   most half the LDS and registers, and keeps a ring of two K stages);
 * the tile must divide M x N, else MX_ERR_SHAPE.  0, 0, 0 picks the tiling
 * as mx_gemm does.  For tuning and for tests that cover every tiling.  The
 * result differs from mx_gemm's only by the binary32 accumulation order of
 * the K steps, i.e. within the GEMM tolerance; with mx_gemm's own tiling it
 * is bitwise mx_gemm's.  Other arguments and errors as mx_gemm.
 */
int mx_gemm_tiled(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales, int64_t M,
                  int64_t N, int64_t K, int fmt, const void* bias, int bias_dtype, void* c, int c_dtype, int64_t ldc,
                  int tile_m, int tile_n, int wg_per_cu, void* stream);

/*
 * mx_gemm_plan -- the launch plan of a dense GEMM: output tile, workgroups
 * per compute unit and K split.  [P3] Tuned GEMMs: a table keyed by the
 * compute-unit count and the GEMM's M, N and K names the kernel (its tile)
 * and a split-K factor for each tuned shape.  Here the table holds the best
 * of a measured sweep over every dense tiling and K split of the Flux-12B
 * block linears (fwd, dgrad, wgrad) at 512 to 4096 tokens, where it beat
 * the rule; any other shape gets the rule of mx_gemm with no split.
 *
 *  M, N, K, fmt     as mx_gemm.
 *  plan             out, int[4]: tile_m, tile_n, wg_per_cu, split_k (the
 *                   arguments mx_gemm_splitk takes).
 *  workspace_bytes  out (may be NULL): the workspace mx_gemm_splitk needs
 *                   for this plan, split_k * M * N * 4 bytes (0 if
 *                   split_k = 1).
 * Host only; nothing is enqueued.  Errors: MX_ERR_NULL (plan NULL),
 * MX_ERR_FORMAT, MX_ERR_SHAPE (M, N or K not multiples of 256).
 */
int mx_gemm_plan(int64_t M, int64_t N, int64_t K, int fmt, int* plan, int64_t* workspace_bytes);

/*
 * mx_gemm_splitk -- mx_gemm with the K range cut into split_k equal parts
 * computed by separate workgroups, then summed in a fixed order.  [P3]
 * Tuned GEMMs (the split-K column of the tuned table): where a GEMM has
 * fewer output tiles than compute units -- few tokens, long K -- the split
 * parts fill the idle ones.
 *
 * The GEMM writes part s (the binary32 product over K elements
 * [s*K/split_k, (s+1)*K/split_k), what mx_gemm_tiled with c_dtype = MX_F32
 * and no bias stores for that K slice) to workspace + s*M*N (row pitch N);
 * a second launch on the same stream then sets
 *   c[m][n] = round(fl32(...fl32(fl32(p_0 + p_1) + p_2)... + p_{S-1}) + bias[n])
 * with one rounding to c_dtype (nearest even for bf16).  The order is fixed
 * and no atomics are used, so repeated calls are bitwise identical; the
 * result differs from mx_gemm's by the binary32 summation order only.
 *
 *  tile_m, tile_n, wg_per_cu   the tiling, as mx_gemm_tiled (0, 0, 0: the
 *               tiling mx_gemm would take).
 *  split_k      1 .. MX_SPLIT_K_MAX; K must be a multiple of 128 * split_k.
 *               split_k = 1 is mx_gemm_tiled (workspace unused).
 *  workspace    device buffer of at least split_k * M * N * 4 bytes,
 *               16-byte aligned, owned by the caller; overwritten; it must
 *               not overlap A, B, bias or C.  Calls that share a workspace
 *               must be ordered (same stream).
 * Other arguments as mx_gemm.  Errors: as mx_gemm_tiled, plus MX_ERR_SHAPE
 * (split_k out of range, K not a multiple of 128 * split_k, workspace too
 * small), MX_ERR_NULL / MX_ERR_ALIGN (workspace missing or misaligned when
 * split_k > 1).
 */
#define MX_SPLIT_K_MAX 16
int mx_gemm_splitk(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales, int64_t M,
                   int64_t N, int64_t K, int fmt, const void* bias, int bias_dtype, void* c, int c_dtype,
                   int64_t ldc, int tile_m, int tile_n, int wg_per_cu, int split_k, void* workspace,
                   int64_t workspace_bytes, void* stream);

/*
 * mx_gemm_many -- several GEMMs of one format in a single launch, with the
 * results of n mx_gemm calls made with each item's arguments (each GEMM
 * takes the tile shape mx_gemm would give it, so the results are bitwise
 * those of mx_gemm).  For a linear layer's forward, data-gradient and
 * weight-gradient GEMMs, which are independent once the operands are packed
 * ([P1] description): one launch lets the compute units that finish one
 * GEMM's tiles start the next GEMM's instead of idling until every tile of
 * the launch is done.  Items of one tile shape share a launch, and so do
 * items of two shapes that run the same number of wavefronts at the same
 * residency (256x192, 192x256, 192x192 and 256x128 at one workgroup per
 * compute unit, pairwise; 256x128 with 128x256 or 192x192 at two); other
 * shapes take launches of their own.
 *
 *  items        host array of n items; each item's fields have the meaning
 *               and rules of the mx_gemm arguments of the same names.  No
 *               item's C may overlap another item's A, B or C.
 *  n            1 <= n <= MX_GEMM_MANY_MAX.
 *  fmt          element format of every operand.
 * Items with M = 0 or N = 0 are skipped.  An item with accumulate = 1 adds
 * into its C as mx_gemm_accumulate does, in a launch of its own after the
 * others (any other value than 0 or 1 is MX_ERR_FORMAT).
 * Errors: MX_ERR_NULL (items NULL), MX_ERR_SHAPE (n out of range), then as
 * mx_gemm for the first failing item; nothing is enqueued on an error.
 */
#define MX_GEMM_MANY_MAX 4
typedef struct {
  mx_packed A, B;
  int64_t M, N, K;
  const void* bias;
  int32_t bias_dtype;
  int32_t c_dtype;
  void* C;
  int64_t ldc;
  int32_t accumulate;     /* 0: C = A . B^T (mx_gemm); 1: C += A . B^T (mx_gemm_accumulate) */
  int32_t reserved;       /* 0 */
} mx_gemm_item;

int mx_gemm_many(const mx_gemm_item* items, int n, int fmt, void* stream);

/* ---------------------------------------------------------------- fused MLP */
/*
 * Fused MX MLP, Y = fc2(GELU_tanh(fc1(X) + b1)) ([P1] description and
 * Summary: one function owns fc1 -> epilogue -> fc2, the packer takes the
 * epilogue as a prologue in both directions, the activation is packed
 * straight from on-chip memory and the pre-activation gradient is never
 * assembled; db1 is finished from the column sums of dh that the packer
 * accumulates).
 * All packs use fmt / scale_mode / hadamard (MXFP6: MX_E2M3, FLOOR, 1).
 * M, D, F multiples of 256.  Packed buffers: rows x K as named.
 * The backward's weight gradients may be the caller's main_grad buffers
 * ([P1] commit messages: the gradient lands in main_grad for both MLP
 * matrices): accumulate_wgrad = 0 overwrites them, 1 adds into them (any
 * other value is MX_ERR_FORMAT).
 */
typedef struct {
  int64_t M, D, F;        /* tokens; fc1 in = fc2 out width; fc1 out = fc2 in width */
  int32_t fmt, scale_mode, hadamard, reserved;
  const void* X;          /* bf16 [M][D] */
  const void* W1;         /* bf16 [F][D] */
  const void* b1;         /* bf16 [F] or NULL */
  const void* W2;         /* bf16 [D][F] */
  void* h;                /* out bf16 [M][F]: fc1 + b1, kept for the backward */
  void* Y;                /* out bf16 [M][D] */
  mx_packed Xr;           /* work: X rows [M] x K=D */
  mx_packed Xc;           /* out (kept): X columns [D] x K=M, for the fc1 weight gradient */
  mx_packed W1r;          /* work: W1 rows [F] x K=D */
  mx_packed W1c;          /* out (kept): W1 columns [D] x K=F, for the fc1 data gradient */
  mx_packed W2r;          /* work: W2 rows [D] x K=F */
  mx_packed W2c;          /* out (kept): W2 columns [F] x K=D, for the fc2 data gradient */
  mx_packed ar;           /* work: a = GELU(h) rows [M] x K=F (a itself is never stored) */
  mx_packed ac;           /* out (kept): a columns [F] x K=M, for the fc2 weight gradient */
} mx_mlp_fwd_args;

typedef struct {
  int64_t M, D, F;
  int32_t fmt, scale_mode, hadamard;
  int32_t accumulate_wgrad; /* 0: dW1, dW2 are overwritten; 1: the weight gradients are added into them
                               (main_grad buffers accumulated over microbatches, as mx_gemm_accumulate) */
  const void* dY;         /* bf16 [M][D] */
  const void* h;          /* bf16 [M][F] from the forward */
  mx_packed Xc, W1c, W2c, ac; /* from the forward */
  void* da;               /* out bf16 [M][F]: fc2 data gradient (materialised) */
  void* dX;               /* out bf16 [M][D] */
  void* dW1;              /* out bf16 [F][D] */
  void* dW2;              /* out bf16 [D][F] */
  float* db1;             /* out fp32 [F], or NULL to skip the bias gradient */
  float* db1_partials;    /* work fp32 [M/32][F]; required when db1 is set */
  mx_packed dYr;          /* work: dY rows [M] x K=D */
  mx_packed dYc;          /* work: dY columns [D] x K=M */
  mx_packed dhr;          /* work: dh = dGELU(da, h) rows [M] x K=F (dh itself is never stored) */
  mx_packed dhc;          /* work: dh columns [F] x K=M */
} mx_mlp_bwd_args;

int mx_fused_mlp_fwd(const mx_mlp_fwd_args* args, void* stream);
int mx_fused_mlp_bwd(const mx_mlp_bwd_args* args, void* stream);

/* ---------------------------------------------------------------- grouped */
/*
 * mx_grouped_gemm -- ragged grouped GEMM over G experts ([P4] commit
 * messages).  offsets: device int32 [G], cumulative group ends: group g owns
 * ragged indices [offsets[g-1], offsets[g]) (offsets[-1] := 0).  Contract
 * (caller invariant): non-decreasing, multiples of 128 ([P4] first commit
 * message: expert sizes are 128-row multiples, which keeps every 32-row
 * quantization block and every tile inside one expert), offsets[G-1] <= R.  Indices at
 * or past offsets[G-1] are neither read nor written.  validate_offsets = 1
 * copies offsets to the host, synchronizing `stream`, and checks them
 * (MX_ERR_OFFSETS).  Counts that are multiples of 256 (the alignment another
 * stack on the pages requires) are a special case and need nothing else.
 * Tiling (RAGGED_M): each group's rows are cut into 256-row tiles (128x256
 * for DSWIGLU), the last one holding 128 rows when the count is an odd
 * multiple of 128; rows of a tile past its group's end are neither read nor
 * stored.
 *
 * MX_GROUPED_RAGGED_M (forward and data gradients):
 *   A [R] x K, B [G][N] x K (expert g's rows at B + g*N rows; its scales
 *   at B.scales + g * mx_scales_bytes(N, K), as written by a batch-G
 *   mx_quantize),
 *   C[r][n] = sum_k A[r][k] * B_g(r)[n][k], bf16 [R][N].  N, K multiples of
 *   256 (SWIGLU: also N/2 a multiple of 128).
 *   epilogue MX_EPI_NONE:    C stored.
 *   epilogue MX_EPI_SWIGLU:  N = 2F; C = H [R][2F] = [gate | up] stored
 *     (the pre-activation kept for the backward); z = SwiGLU(H) is
 *     quantized in the epilogue (fmt, scale_mode) into out_row = z rows [R]
 *     x K=F and out_col = z columns [F] x K=R.  z itself is never stored.
 *   epilogue MX_EPI_DSWIGLU: N = F; the GEMM result is dz; with H [R][2F]
 *     (aux), dH = dSwiGLU(dz, H) is quantized into out_row = dH rows [R] x
 *     K=2F and out_col = dH columns [2F] x K=R.  C (bf16 dz [R][F]) may be
 *     NULL; dz and dH are otherwise never stored.
 * MX_GROUPED_RAGGED_K (weight gradients):
 *   A [M] x K=R, B [N] x K=R, C bf16 [G][M][N]:
 *   C_g = sum over k in group g of A[:, k] B[:, k]^T; an empty group's C_g
 *   is written as zeros.  M, N multiples of 256.
 * Errors: as mx_gemm, plus MX_ERR_OFFSETS; G <= 0 is MX_ERR_SHAPE; R == 0
 * enqueues nothing except, in RAGGED_K mode, the zero fill of C.
 */
typedef struct {
  int32_t mode;            /* mx_grouped_mode */
  int32_t epilogue;        /* mx_epilogue (RAGGED_M only) */
  int32_t fmt;             /* element format of A, B and the epilogue's outputs */
  int32_t scale_mode;      /* scale selection of the epilogue's quantization */
  int32_t G;               /* number of groups, >= 1 */
  int32_t validate_offsets;
  int64_t R;               /* ragged extent: rows (RAGGED_M) or K (RAGGED_K) allocated */
  int64_t M, N, K;         /* RAGGED_M: N, K used (M ignored); RAGGED_K: M, N used (K ignored) */
  const int32_t* offsets;  /* device int32 [G] */
  mx_packed A, B;
  void* C;                 /* bf16 output, see mode */
  const void* aux;         /* DSWIGLU: H bf16 [R][2F] */
  mx_packed out_row, out_col; /* epilogue quantization outputs */
} mx_grouped_args;

int mx_grouped_gemm(const mx_grouped_args* args, void* stream);

/* ---------------------------------------------------------------- misc */
/* Human-readable name of a status code (static string). */
const char* mx_status_str(int status);
/* 1 if HIP device `device` is a gfx950 (MI355X-class) GPU, else 0. */
int mx_device_supported(int device);
/* Bytes of one packed operand's codes / blocked scales for rows x K in fmt (0 on bad input):
 * ceil(K/128) * rows * 16 * bits and ceil(K/128) * rows * 4. */
int64_t mx_codes_bytes(int fmt, int64_t rows, int64_t K);
int64_t mx_scales_bytes(int64_t rows, int64_t K);
/* Library version string. */
const char* mx_version(void);
/* Measurement helper: enqueue on `stream` one wavefront that spins for
 * `microseconds` of wall-clock time (1 .. 10^6) and writes, to the device
 * array out[2] (16-byte aligned), the shader-clock cycles (s_memtime) and
 * the wall-clock ticks (s_memrealtime, mx_wall_clock_khz() kHz) it saw:
 * the shader clock in kHz is out[0] / out[1] * mx_wall_clock_khz().  Run
 * beside another stream's kernels, it reads the clock they run at (which
 * operand data can pull below the rated 2.4 GHz).  The wait is bounded by
 * the wall clock.  Errors: MX_ERR_NULL, MX_ERR_ALIGN, MX_ERR_SHAPE,
 * MX_ERR_DEVICE, MX_ERR_LAUNCH. */
int mx_clock_sample(int64_t microseconds, uint64_t* out, void* stream);
/* Wall-clock rate of the current device in kHz (0 if unknown). */
int64_t mx_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* MX_H */
