// Block-scaled MX GEMM for gfx950: C = A . B^T on K-major packed operands,
// on the CDNA4 scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4: E8M0
// block scales applied inside the instruction, binary32 accumulation).
//
// [P1] "feat(mxfp6): MXFP6 (E2M3) Flux linears, a fused MLP, and the MLPerf
//      recipe": MXFP6 GEMMs for forward, dgrad and wgrad, bias added in the
//      store epilogue into the fp32 accumulator (description, commit
//      messages).
// [P3] "MXFP4 training for Flux models": MXFP4 GEMM, NT layout
//      (Troubleshooting).
// [P4] "MXFP8 cudnn-fe Swiglu fused Grouped MLP fwd/bwd and wgrad group
//      gemm": ragged grouped GEMM with the expert picked from the tile
//      coordinate (counts are multiples of 128, so no tile straddles two
//      experts), SwiGLU / dSwiGLU epilogues that quantize rowwise 1x32 and
//      columnwise 32x1 in the same launch, ragged-K weight gradient writing
//      zeros for empty experts (commit messages).
//
// Tiling.  512 threads = 8 wavefronts in a 2 (M) x 4 (N) grid over a
// BM x 256 output tile (BM = 256 or 128); each wavefront owns a
// (BM/2) x 64 sub-tile = (BM/64) x 2 MFMA tiles of 32 x 32.  K advances 128
// elements per stage; A and B stages sit in LDS (row pitch = stage bytes +
// 16, which spreads consecutive rows over distinct LDS banks for the 16-byte
// operand reads), double-buffered, with the next stage's global loads in
// flight while the current one is multiplied.
//
// MFMA operand layout (measured): lane l holds row l%32 of A (of B) and the
// 32-element K block g = l/32 of the 64-element step.  E2M1 / E2M3 take the
// block's 32 codes contiguously (16 / 24 bytes); E4M3 takes K [16g, 16g+16)
// in bytes 0-15 and [32+16g, 32+16g+16) in bytes 16-31.  The lane's scale
// operand is the E8M0 byte of (its row, block g).  The 16 accumulators of
// lane l hold C rows 8*(i/4) + 4*(l/32) + i%4, column l%32.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kBK = 128;
constexpr int kBN = 256;

template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<kE4M3> { static constexpr int kCode = 0; };
template <> struct MfmaFmt<kE2M3> { static constexpr int kCode = 2; };
template <> struct MfmaFmt<kE2M1> { static constexpr int kCode = 4; };

template <int FMT, int BM, int EPI>
struct Cfg {
  static constexpr int kBits = FmtTraits<FMT>::kBits;
  static constexpr int kRowBytes = kBK * kBits / 8;  // 64 / 96 / 128
  static constexpr int kPitch = kRowBytes + 16;
  static constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per row per stage
  static constexpr int kAOff = 0;
  static constexpr int kBOff = BM * kPitch;
  static constexpr int kASOff = kBOff + kBN * kPitch;
  static constexpr int kBSOff = kASOff + BM * 4;
  static constexpr int kStage = kBSOff + kBN * 4;
  static constexpr int kMI = BM / 64;  // MFMA tiles per wavefront along M
  static constexpr int kNJ = 2;        // along N
  static constexpr int kAIters = (BM * kChunks + kThreads - 1) / kThreads;
  static constexpr int kBIters = (kBN * kChunks + kThreads - 1) / kThreads;
  // epilogue staging
  static constexpr int kZPitch = 128 * 2 + 16;  // SwiGLU: z tile BM x 128 bf16
  static constexpr int kDPitch = kBN * 2 + 16;  // dSwiGLU: two BM x 256 bf16 tiles
  static constexpr int kEpiBytes = EPI == kEpiSwiglu ? BM * kZPitch : (EPI == kEpiDSwiglu ? 2 * BM * kDPitch : 0);
  static constexpr int kSmem = (2 * kStage > kEpiBytes) ? 2 * kStage : kEpiBytes;
};

// Read one lane's A/B operand for K step ks (0 or 1) of the stage from a row
// of the LDS tile.
template <int FMT>
__device__ __forceinline__ v8i lds_operand(const uint8_t* rowp, int ks, int g) {
  v8i r;
  if constexpr (FMT == kE4M3) {
    const v4i a = *reinterpret_cast<const v4i*>(rowp + ks * 64 + 16 * g);
    const v4i b = *reinterpret_cast<const v4i*>(rowp + ks * 64 + 32 + 16 * g);
    r = v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  } else if constexpr (FMT == kE2M1) {
    const v4i a = *reinterpret_cast<const v4i*>(rowp + ks * 32 + 16 * g);
    r = v8i{a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  } else {
    const uint8_t* q = rowp + ks * 48 + 24 * g;
    const v2i a = *reinterpret_cast<const v2i*>(q);
    const v2i b = *reinterpret_cast<const v2i*>(q + 8);
    const v2i c = *reinterpret_cast<const v2i*>(q + 16);
    r = v8i{a.x, a.y, b.x, b.y, c.x, c.y, 0, 0};
  }
  return r;
}

template <int FMT, int BM, int MODE, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p) {
  using CF = Cfg<FMT, BM, EPI>;
  constexpr int kBits = CF::kBits;
  __shared__ __attribute__((aligned(16))) uint8_t smem[CF::kSmem];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lrow = lane & 31, g = lane >> 5;

  // ---------------------------------------------------------------- tile
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;  // SwiGLU: blockIdx.x indexes 128-column z blocks
  int64_t kbeg = 0, kend = p.K;
  int64_t b_row0 = 0;           // first B row of this tile's group
  int64_t c_off = 0;            // element offset of this tile's group in C
  if constexpr (MODE == kRaggedM) {
    // offsets are a caller invariant; clamping keeps every access inside the
    // buffers even if it is broken
    int64_t end = p.offsets[p.G - 1];
    end = end < p.R ? end : p.R;
    if (m0 >= end) return;  // rows at or past the last group end: untouched
    int gi = 0;
    while (p.offsets[gi] <= m0) ++gi;
    b_row0 = (int64_t)gi * p.b_group_rows;
  }
  if constexpr (MODE == kRaggedK) {
    const int gi = blockIdx.z;
    kbeg = gi ? p.offsets[gi - 1] : 0;
    kend = p.offsets[gi];
    kbeg = (kbeg < 0 ? 0 : (kbeg > p.R ? p.R : kbeg)) & ~(int64_t)127;
    kend = (kend < 0 ? 0 : (kend > p.R ? p.R : kend)) & ~(int64_t)127;
    if (kend < kbeg) kend = kbeg;
    c_off = (int64_t)gi * p.M * p.N;
  }
  const int64_t row_bytes = p.ktot * kBits / 8;
  const int64_t srow = p.ktot / 32;
  const int nk = (int)((kend - kbeg) / kBK);

  // LDS row r of the B tile -> global B row
  auto b_row = [&](int r) -> int64_t {
    if constexpr (EPI == kEpiSwiglu) {
      const int64_t zb = (int64_t)blockIdx.x * 128;
      return b_row0 + (r < 128 ? zb + r : p.F + zb + (r - 128));
    } else {
      return b_row0 + n0 + r;
    }
  };

  // ---------------------------------------------------------------- loads
  uint4 ra[CF::kAIters], rb[CF::kBIters];
  uint32_t rs = 0;
  auto gload = [&](int64_t k0) {
    const int64_t kb = k0 * kBits / 8;
#pragma unroll
    for (int i = 0; i < CF::kAIters; ++i) {
      const int q = t + kThreads * i;
      if (q < BM * CF::kChunks) {
        const int r = q / CF::kChunks, ch = q % CF::kChunks;
        ra[i] = *reinterpret_cast<const uint4*>(p.a_codes + (m0 + r) * row_bytes + kb + ch * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < CF::kBIters; ++i) {
      const int q = t + kThreads * i;
      if (q < kBN * CF::kChunks) {
        const int r = q / CF::kChunks, ch = q % CF::kChunks;
        rb[i] = *reinterpret_cast<const uint4*>(p.b_codes + b_row(r) * row_bytes + kb + ch * 16);
      }
    }
    if (t < BM) {
      rs = *reinterpret_cast<const uint32_t*>(p.a_scales + (m0 + t) * srow + k0 / 32);
    } else if (t < BM + kBN) {
      rs = *reinterpret_cast<const uint32_t*>(p.b_scales + b_row(t - BM) * srow + k0 / 32);
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* s = smem + buf * CF::kStage;
#pragma unroll
    for (int i = 0; i < CF::kAIters; ++i) {
      const int q = t + kThreads * i;
      if (q < BM * CF::kChunks) {
        const int r = q / CF::kChunks, ch = q % CF::kChunks;
        *reinterpret_cast<uint4*>(s + CF::kAOff + r * CF::kPitch + ch * 16) = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < CF::kBIters; ++i) {
      const int q = t + kThreads * i;
      if (q < kBN * CF::kChunks) {
        const int r = q / CF::kChunks, ch = q % CF::kChunks;
        *reinterpret_cast<uint4*>(s + CF::kBOff + r * CF::kPitch + ch * 16) = rb[i];
      }
    }
    if (t < BM) {
      *reinterpret_cast<uint32_t*>(s + CF::kASOff + t * 4) = rs;
    } else if (t < BM + kBN) {
      *reinterpret_cast<uint32_t*>(s + CF::kBSOff + (t - BM) * 4) = rs;
    }
  };

  // ---------------------------------------------------------------- main loop
  v16f acc[CF::kMI][CF::kNJ];
#pragma unroll
  for (int i = 0; i < CF::kMI; ++i)
#pragma unroll
    for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // LDS rows this lane reads
  int arow[CF::kMI], brow[CF::kNJ];
#pragma unroll
  for (int i = 0; i < CF::kMI; ++i) arow[i] = wm * (BM / 2) + 32 * i + lrow;
#pragma unroll
  for (int j = 0; j < CF::kNJ; ++j)
    brow[j] = (EPI == kEpiSwiglu) ? (128 * j + 32 * wn + lrow) : (64 * wn + 32 * j + lrow);

  if (nk > 0) {
    gload(kbeg);
    lstore(0);
    __syncthreads();
  }
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) gload(kbeg + (int64_t)(it + 1) * kBK);
    const uint8_t* s = smem + cur * CF::kStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i af[CF::kMI], bf[CF::kNJ];
      int sa[CF::kMI], sb[CF::kNJ];
#pragma unroll
      for (int i = 0; i < CF::kMI; ++i) {
        af[i] = lds_operand<FMT>(s + CF::kAOff + arow[i] * CF::kPitch, ks, g);
        sa[i] = (int)(*reinterpret_cast<const uint32_t*>(s + CF::kASOff + arow[i] * 4) >> (8 * (2 * ks + g)));
      }
#pragma unroll
      for (int j = 0; j < CF::kNJ; ++j) {
        bf[j] = lds_operand<FMT>(s + CF::kBOff + brow[j] * CF::kPitch, ks, g);
        sb[j] = (int)(*reinterpret_cast<const uint32_t*>(s + CF::kBSOff + brow[j] * 4) >> (8 * (2 * ks + g)));
      }
#pragma unroll
      for (int i = 0; i < CF::kMI; ++i)
#pragma unroll
        for (int j = 0; j < CF::kNJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[i], bf[j], acc[i][j], MfmaFmt<FMT>::kCode, MfmaFmt<FMT>::kCode, 0, sa[i], 0, sb[j]);
    }
    if (it + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == kEpiStore) {
#pragma unroll
    for (int j = 0; j < CF::kNJ; ++j) {
      const int64_t n = n0 + 64 * wn + 32 * j + lrow;
      float bias = 0.0f;
      if (p.bias) {
        bias = p.bias_f32 ? reinterpret_cast<const float*>(p.bias)[n]
                          : bf16_to_f32(reinterpret_cast<const uint16_t*>(p.bias)[n]);
      }
#pragma unroll
      for (int i = 0; i < CF::kMI; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + wm * (BM / 2) + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
          const float v = acc[i][j][e] + bias;
          const int64_t idx = c_off + m * p.ldc + n;
          if (p.c_f32) reinterpret_cast<float*>(p.c)[idx] = v;
          else reinterpret_cast<uint16_t*>(p.c)[idx] = (uint16_t)f32_to_bf16(v);
        }
      }
    }
  } else if constexpr (EPI == kEpiSwiglu) {
    // Lane holds gate (j = 0) and up (j = 1) of the same (row, z column).
    // H [R][2F] is stored; z = SwiGLU(bf16 gate, bf16 up) goes to LDS only.
    uint8_t* zt = smem;
    const int64_t zb = (int64_t)blockIdx.x * 128;
    const int zc = 32 * wn + lrow;
    uint16_t* H = reinterpret_cast<uint16_t*>(p.c);
#pragma unroll
    for (int i = 0; i < CF::kMI; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ml = wm * (BM / 2) + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
        const int64_t m = m0 + ml;
        const float hg = round_bf16(acc[i][0][e]);
        const float hu = round_bf16(acc[i][1][e]);
        H[m * 2 * p.F + zb + zc] = (uint16_t)f32_to_bf16(hg);
        H[m * 2 * p.F + p.F + zb + zc] = (uint16_t)f32_to_bf16(hu);
        reinterpret_cast<uint16_t*>(zt + ml * CF::kZPitch)[zc] = (uint16_t)f32_to_bf16(swiglu_bf16(hg, hu));
      }
    }
    __syncthreads();
    constexpr int QB = FmtTraits<FMT>::kBits;
    // row blocks: BM rows x 4 blocks of 32 z columns
    for (int q = t; q < BM * 4; q += kThreads) {
      const int row = q >> 2, blk = q & 3;
      float v[32];
      lds_row_block(zt, CF::kZPitch, row, blk * 32, v);
      const int64_t m = m0 + row, col = zb + 32 * blk;
      if (p.q_mode == kRceil)
        quant_store<FMT, kRceil, 0>(v, p.q_row_codes + m * (p.F * QB / 8) + col * QB / 8,
                                    p.q_row_scales + m * (p.F / 32) + col / 32);
      else
        quant_store<FMT, kFloor, 0>(v, p.q_row_codes + m * (p.F * QB / 8) + col * QB / 8,
                                    p.q_row_scales + m * (p.F / 32) + col / 32);
    }
    // column blocks: 128 z columns x BM/32 row blocks (transposed operand)
    for (int q = t; q < 128 * (BM / 32); q += kThreads) {
      const int col = q & 127, rb2 = q >> 7;
      float v[32];
      lds_col_block(zt, CF::kZPitch, rb2 * 32, col, v);
      const int64_t cz = zb + col, m = m0 + 32 * rb2;
      if (p.q_mode == kRceil)
        quant_store<FMT, kRceil, 0>(v, p.q_col_codes + cz * (p.R * QB / 8) + m * QB / 8,
                                    p.q_col_scales + cz * (p.R / 32) + m / 32);
      else
        quant_store<FMT, kFloor, 0>(v, p.q_col_codes + cz * (p.R * QB / 8) + m * QB / 8,
                                    p.q_col_scales + cz * (p.R / 32) + m / 32);
    }
  } else {  // kEpiDSwiglu
    // dz = bf16(acc); with H: d_gate -> tile 0, d_up -> tile 1 (LDS only).
    uint8_t* tg = smem;
    uint8_t* tu = smem + BM * CF::kDPitch;
    const uint16_t* H = p.aux;
#pragma unroll
    for (int j = 0; j < CF::kNJ; ++j) {
      const int nl = 64 * wn + 32 * j + lrow;
      const int64_t n = n0 + nl;
#pragma unroll
      for (int i = 0; i < CF::kMI; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ml = wm * (BM / 2) + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
          const int64_t m = m0 + ml;
          const float dz = round_bf16(acc[i][j][e]);
          if (p.c) reinterpret_cast<uint16_t*>(p.c)[m * p.F + n] = (uint16_t)f32_to_bf16(dz);
          const float gv = bf16_to_f32(H[m * 2 * p.F + n]);
          const float uv = bf16_to_f32(H[m * 2 * p.F + p.F + n]);
          reinterpret_cast<uint16_t*>(tg + ml * CF::kDPitch)[nl] = (uint16_t)f32_to_bf16(dswiglu_gate_bf16(dz, gv, uv));
          reinterpret_cast<uint16_t*>(tu + ml * CF::kDPitch)[nl] = (uint16_t)f32_to_bf16(dswiglu_up_bf16(dz, gv));
        }
      }
    }
    __syncthreads();
    constexpr int QB = FmtTraits<FMT>::kBits;
    const int64_t W = 2 * p.F;  // dH width
    for (int q = t; q < 2 * BM * 8; q += kThreads) {
      const int half = q / (BM * 8), rq = q % (BM * 8);
      const int row = rq >> 3, blk = rq & 7;
      float v[32];
      lds_row_block(half ? tu : tg, CF::kDPitch, row, blk * 32, v);
      const int64_t m = m0 + row, col = (half ? p.F : 0) + n0 + 32 * blk;
      if (p.q_mode == kRceil)
        quant_store<FMT, kRceil, 0>(v, p.q_row_codes + m * (W * QB / 8) + col * QB / 8,
                                    p.q_row_scales + m * (W / 32) + col / 32);
      else
        quant_store<FMT, kFloor, 0>(v, p.q_row_codes + m * (W * QB / 8) + col * QB / 8,
                                    p.q_row_scales + m * (W / 32) + col / 32);
    }
    for (int q = t; q < 2 * kBN * (BM / 32); q += kThreads) {
      const int half = q / (kBN * (BM / 32)), cq = q % (kBN * (BM / 32));
      const int col = cq % kBN, rb2 = cq / kBN;
      float v[32];
      lds_col_block(half ? tu : tg, CF::kDPitch, rb2 * 32, col, v);
      const int64_t cw = (half ? p.F : 0) + n0 + col, m = m0 + 32 * rb2;
      if (p.q_mode == kRceil)
        quant_store<FMT, kRceil, 0>(v, p.q_col_codes + cw * (p.R * QB / 8) + m * QB / 8,
                                    p.q_col_scales + cw * (p.R / 32) + m / 32);
      else
        quant_store<FMT, kFloor, 0>(v, p.q_col_codes + cw * (p.R * QB / 8) + m * QB / 8,
                                    p.q_col_scales + cw * (p.R / 32) + m / 32);
    }
  }
}

template <int FMT, int BM, int MODE, int EPI>
hipError_t launch_one(const GemmParams& p, hipStream_t stream) {
  dim3 grid;
  if (MODE == kDense) {
    grid = dim3((unsigned)(p.N / kBN), (unsigned)(p.M / BM), 1);
  } else if (MODE == kRaggedM) {
    const unsigned nt = EPI == kEpiSwiglu ? (unsigned)(p.F / 128) : (unsigned)(p.N / kBN);
    grid = dim3(nt, (unsigned)(p.R / BM), 1);
  } else {
    grid = dim3((unsigned)(p.N / kBN), (unsigned)(p.M / BM), (unsigned)p.G);
  }
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<FMT, BM, MODE, EPI>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const GemmParams& p, int mode, int epi, hipStream_t stream) {
  if (mode == kDense) return launch_one<FMT, 128, kDense, kEpiStore>(p, stream);
  if (mode == kRaggedM) {
    if (epi == kEpiSwiglu) return launch_one<FMT, 128, kRaggedM, kEpiSwiglu>(p, stream);
    if (epi == kEpiDSwiglu) return launch_one<FMT, 128, kRaggedM, kEpiDSwiglu>(p, stream);
    return launch_one<FMT, 128, kRaggedM, kEpiStore>(p, stream);
  }
  return launch_one<FMT, 128, kRaggedK, kEpiStore>(p, stream);
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, int fmt, int mode, int epi, hipStream_t stream) {
  switch (fmt) {
    case kE2M1: return launch_fmt<kE2M1>(p, mode, epi, stream);
    case kE2M3: return launch_fmt<kE2M3>(p, mode, epi, stream);
    case kE4M3: return launch_fmt<kE4M3>(p, mode, epi, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mx
