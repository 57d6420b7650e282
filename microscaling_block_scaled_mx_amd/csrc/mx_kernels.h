// Internal launch interface between the C ABI (mx_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Blocked E8M0 scale layout of a packed operand with `rows` rows and K
// elements per row: the four scale bytes of one 128-element K group form a
// dword (block 4q+i in byte i), and the dwords of one K group are stored row
// after row -- [ceil(K/128)][rows][4] bytes.  A GEMM stage then reads the
// scales of a row panel as one contiguous run.  Pad bytes of a last, partial
// K group are written as 0.
__host__ __device__ __forceinline__ int64_t scale_offset(int64_t row, int64_t blk, int64_t rows) {
  return ((blk >> 2) * rows + row) * 4 + (blk & 3);
}
__host__ __device__ __forceinline__ int64_t scale_bytes(int64_t rows, int64_t K) {
  return ((K / 32 + 3) / 4) * rows * 4;
}

// Codes use the same K-group-major order: the codes of one row's 128-element
// K group take 16 * bits contiguous bytes, and the groups of one K group are
// stored row after row -- [ceil(K/128)][rows][16 * bits] bytes.  A GEMM
// stage then reads a row panel's codes as one contiguous run.  Inside a
// group, E2M1 and E4M3 blocks (32 codes, 16 / 32 bytes) follow each other;
// an E2M3 block (24 bytes) is split so that each MFMA operand is one 16-byte
// and one 8-byte read: block b's first 16 bytes at 16 b, its last 8 bytes
// at 64 + 8 (b ^ s), s = bit 4 of the row.  Pad bytes of a partial last
// group are 0.
// Byte offset of the group holding element k (any k) of a row:
__host__ __device__ __forceinline__ int64_t code_group(int64_t row, int64_t k, int64_t rows, int bits) {
  return ((k >> 7) * rows + row) * (16 * bits);
}
__host__ __device__ __forceinline__ int64_t code_bytes(int64_t rows, int64_t K, int bits) {
  return ((K + 127) / 128) * rows * (16 * bits);
}


struct PackParams {
  const uint16_t* x;    // prologue input (bf16 bits)
  const uint16_t* aux;  // second prologue input or nullptr
  int64_t R, C;         // logical quantized tensor [R][C] per batch entry
  uint8_t* row_codes;   // K-group-major codes, rows R, K = C, or nullptr
  uint8_t* row_scales;  // blocked layout, rows R, K = C
  uint8_t* col_codes;   // K-group-major codes, rows C, K = R, or nullptr
  uint8_t* col_scales;  // blocked layout, rows C, K = R
  float* partials;      // [R/32][C] or nullptr
  uint64_t sr_seed;     // stochastic-rounding kernels only: Philox key
  int64_t batch;        // batch entries (set by launch_pack)
};

// Up to kPackManyMax tensors packed in one launch: item i owns workgroups
// first[i] .. first[i + 1] - 1 (ceil(C/128) * ceil(R/128) * batch of them).
constexpr int kPackManyMax = 8;
struct PackMany {
  PackParams p[kPackManyMax];
  int64_t first[kPackManyMax + 1];
  int n;
};

// Compute units of the current device (cached per device).
int cu_count();

bool pack_supported(int fmt, int mode, int had, int pro);
hipError_t launch_pack(const PackParams& p, int fmt, int mode, int had, int pro, int64_t batch,
                       hipStream_t stream);
hipError_t launch_pack_many(const PackMany& m, int fmt, int mode, int had, int pro, hipStream_t stream);
// MXFP4 (E2M1, FLOOR, no rotation, identity prologue) with stochastic rounding
hipError_t launch_pack_sr(const PackParams& p, int64_t batch, hipStream_t stream);
hipError_t launch_colsum_finish(const float* partials, int64_t nb, int64_t C, float* out, int64_t batch,
                                hipStream_t stream);

enum GemmMode { kDense = 0, kRaggedM = 1, kRaggedK = 2 };
// kEpiAccum (dense only): the store of kEpiStore, adding into the previous C.
// kEpiSplit (dense only): the K range cut into split_k parts, each stored in
// binary32 without the bias (see GemmParams::split_k).
enum Epilogue { kEpiStore = 0, kEpiSwiglu = 1, kEpiDSwiglu = 2, kEpiAccum = 3, kEpiSplit = 4 };

struct GemmParams {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int64_t M, N;          // output extent (per group for ragged-K)
  int64_t K;             // reduction length (dense, ragged-M)
  int64_t ktot;          // row length of A/B in elements (K, or R for ragged-K)
  const void* bias;      // [N] or nullptr
  int bias_f32;          // bias dtype: 0 bf16, 1 f32
  void* c;               // output
  int64_t ldc;           // output row pitch in elements
  int c_f32;             // output dtype: 0 bf16, 1 f32
  // grouped
  const int32_t* offsets;
  int G;
  int64_t b_group_rows;  // ragged-M: rows of B per group (N)
  // epilogue quantization (SwiGLU / dSwiGLU)
  int64_t R;             // ragged extent allocated (rows of H / out_row, K of out_col)
  int64_t F;             // SwiGLU hidden width
  const uint16_t* aux;   // dSwiGLU: H [R][2F]
  uint8_t* q_row_codes;
  uint8_t* q_row_scales;
  uint8_t* q_col_codes;
  uint8_t* q_col_scales;
  int q_mode;            // scale mode for the epilogue's quantization
  // dense: 0 lets the launch pick the output tile shape; 1 + i forces entry
  // i of the dense shape table (see dense_tile_index)
  int tile_shape;
  // kEpiSplit: the K range cut into split_k >= 2 equal parts; part s is
  // computed by its own workgroups into C + s * M * ldc (binary32, no bias),
  // for launch_splitk_reduce to sum
  int split_k;
};

hipError_t launch_gemm(const GemmParams& p, int fmt, int mode, int epi, hipStream_t stream);
// c[m][n] = round(((ws_0 + ws_1) + ... + ws_{S-1}) + bias[n]) over the
// split_k binary32 partial results ws_s = ws + s * M * N (row pitch N), in
// that order, rounded once to bf16 (nearest even) or stored as binary32.
hipError_t launch_splitk_reduce(const float* ws, int split_k, int64_t M, int64_t N, const void* bias, int bias_f32,
                                void* c, int c_f32, int64_t ldc, hipStream_t stream);

// A dense GEMM's launch plan: output tile, workgroups per compute unit and
// K split.  plan_gemm gives the measured best of the tuned table for this
// compute-unit count, format and M x N x K, else the rounds x tile-area
// rule with no split; split_k > 1 needs a workspace of split_k * M * N
// binary32 values.
struct GemmPlan {
  int tile_m, tile_n, wg_per_cu, split_k;
};
bool plan_gemm(int fmt, int64_t M, int64_t N, int64_t K, GemmPlan* out);
// Index of the dense output tile shape bm x bn at wg_per_cu workgroups per
// compute unit for an M x N output, or -1 if it is not one of the dense
// shapes or does not divide M x N.
int dense_tile_index(int bm, int bn, int wg_per_cu, int64_t M, int64_t N);

// Up to kGemmManyMax dense GEMMs (kDense, kEpiStore) of one format in one
// launch; each takes the tile shape launch_gemm would give it.  shape and
// first are filled in by the launch.
constexpr int kGemmManyMax = 4;
struct GemmMany {
  GemmParams p[kGemmManyMax];
  int shape[kGemmManyMax];
  int first[kGemmManyMax + 1];
  int n;
};
hipError_t launch_gemm_many(GemmMany m, int fmt, hipStream_t stream);

}  // namespace mx
