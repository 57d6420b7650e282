// MX packer for gfx950: prologue -> [Hadamard-32] -> amax -> E8M0 -> cast ->
// bit-pack, rowwise (1x32 along dim 1) and/or columnwise (32x1 along dim 0,
// written transposed as a K-major operand), plus per-32-row-block column sums.
//
// [P1] "feat(mxfp6): MXFP6 (E2M3) Flux linears, a fused MLP, and the MLPerf
//      recipe": the packer carries the rotation, takes the activation
//      epilogue as a prologue, and returns column-sum partials for the bias
//      gradient (description, commit messages).
// [P4] "MXFP8 cudnn-fe Swiglu fused Grouped MLP fwd/bwd and wgrad group
//      gemm": rowwise 1x32 and columnwise 32x1 quantization, RCEIL scales,
//      NaN-propagating amax (commit messages).
//
// Work split.  One 256-thread workgroup owns a 64-row x 128-column tile.
//  1. Load: each thread reads four 16-byte chunks (8 bf16) -- a row of the
//     tile is 16 chunks, so a wavefront covers 4 rows x 256 B per load, fully
//     coalesced -- applies the prologue in registers, rounds to bf16 and
//     writes the tile to LDS.  The prologue output exists only on chip.
//  2. Row pass: thread t quantizes the 1x32 block (row t/4, block t%4).
//  3. Column pass: thread t quantizes the 32x1 block (column t%128, row block
//     t/128); adjacent lanes hold adjacent columns, so the LDS reads are
//     conflict-free; its codes land in row (c0 + column) of the transposed
//     operand.
// Rows/columns past R/C (multiples of 32) are masked per chunk.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kTileR = 64, kTileC = 128;
constexpr int kPitch = kTileC * 2 + 16;  // bytes per LDS row (16 B pad)

struct Chunk8 {
  uint32_t w[4];  // 8 bf16, element 2i in the low half of w[i]
};

__device__ __forceinline__ Chunk8 ld_chunk(const uint16_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  Chunk8 c;
  c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  return c;
}

template <int PRO>
__device__ __forceinline__ Chunk8 prologue_chunk(const PackParams& p, const uint16_t* xb, const uint16_t* ab,
                                                 int64_t r, int64_t c) {
  Chunk8 out;
  if constexpr (PRO == kIdentity) {
    out = ld_chunk(xb + r * p.C + c);
  } else if constexpr (PRO == kGelu) {
    Chunk8 h = ld_chunk(xb + r * p.C + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = f32_to_bf16(gelu_bf16(bf16_lo(h.w[i])));
      uint32_t hi = f32_to_bf16(gelu_bf16(bf16_hi(h.w[i])));
      out.w[i] = lo | (hi << 16);
    }
  } else if constexpr (PRO == kDGelu) {
    Chunk8 d = ld_chunk(xb + r * p.C + c);
    Chunk8 h = ld_chunk(ab + r * p.C + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = f32_to_bf16(dgelu_bf16(bf16_lo(d.w[i]), bf16_lo(h.w[i])));
      uint32_t hi = f32_to_bf16(dgelu_bf16(bf16_hi(d.w[i]), bf16_hi(h.w[i])));
      out.w[i] = lo | (hi << 16);
    }
  } else if constexpr (PRO == kSwiglu) {
    // x = H [R][2C] = [gate | up]
    Chunk8 g = ld_chunk(xb + r * 2 * p.C + c);
    Chunk8 u = ld_chunk(xb + r * 2 * p.C + p.C + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = f32_to_bf16(swiglu_bf16(bf16_lo(g.w[i]), bf16_lo(u.w[i])));
      uint32_t hi = f32_to_bf16(swiglu_bf16(bf16_hi(g.w[i]), bf16_hi(u.w[i])));
      out.w[i] = lo | (hi << 16);
    }
  } else {  // kDSwiglu: C = 2F, x = dz [R][F], aux = H [R][2F]
    const int64_t F = p.C / 2;
    const bool gate = c < F;
    const int64_t j = gate ? c : c - F;
    Chunk8 dz = ld_chunk(xb + r * F + j);
    Chunk8 g = ld_chunk(ab + r * p.C + j);
    Chunk8 u = ld_chunk(ab + r * p.C + F + j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo, hi;
      if (gate) {
        lo = dswiglu_gate_bf16(bf16_lo(dz.w[i]), bf16_lo(g.w[i]), bf16_lo(u.w[i]));
        hi = dswiglu_gate_bf16(bf16_hi(dz.w[i]), bf16_hi(g.w[i]), bf16_hi(u.w[i]));
      } else {
        lo = dswiglu_up_bf16(bf16_lo(dz.w[i]), bf16_lo(g.w[i]));
        hi = dswiglu_up_bf16(bf16_hi(dz.w[i]), bf16_hi(g.w[i]));
      }
      out.w[i] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
    }
  }
  return out;
}

template <int FMT, int MODE, int HAD, int PRO>
__global__ __launch_bounds__(256) void pack_kernel(PackParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileR * kPitch];
  constexpr int B = FmtTraits<FMT>::kBits;
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * kTileR, c0 = (int64_t)blockIdx.x * kTileC;
  const int64_t z = blockIdx.z;
  // per-problem bases
  const int64_t in_cols = (PRO == kSwiglu) ? 2 * p.C : (PRO == kDSwiglu ? p.C / 2 : p.C);
  const uint16_t* xb = p.x + z * p.R * in_cols;
  const uint16_t* ab = p.aux ? p.aux + z * p.R * p.C : nullptr;

  // 1. load + prologue -> LDS
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 4, ch = q & 15;
    const int64_t r = r0 + row, c = c0 + ch * 8;
    Chunk8 v;
    if (r < p.R && c < p.C) {
      v = prologue_chunk<PRO>(p, xb, ab, r, c);
    } else {
      v.w[0] = v.w[1] = v.w[2] = v.w[3] = 0u;
    }
    *reinterpret_cast<uint4*>(tile + row * kPitch + ch * 16) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
  }
  __syncthreads();

  // 2. row pass: block (row t/4, blk t%4) along dim 1
  if (p.row_codes) {
    const int row = t >> 2, blk = t & 3;
    const int64_t r = r0 + row, c = c0 + blk * 32;
    uint8_t* scales = p.row_scales + z * scale_bytes(p.R, p.C) + scale_offset(r, c / 32, p.R);
    if (r < p.R && c < p.C) {
      float v[32];
      lds_row_block(tile, kPitch, row, blk * 32, v);
      uint8_t* codes = p.row_codes + z * p.R * (p.C * B / 8) + r * (p.C * B / 8) + c * B / 8;
      quant_store<FMT, MODE, HAD>(v, codes, scales);
    } else if (r < p.R) {
      *scales = 0;  // pad byte of the row's last scale dword (the tile spans exactly one dword)
    }
  }

  // 3. column pass: block (column t%128, rows 32*(t/128) .. +31) along dim 0
  if (p.col_codes || p.partials) {
    const int col = t & 127, blk = t >> 7;
    const int64_t c = c0 + col, r = r0 + blk * 32;
    if (c < p.C) {
      // pad bytes of the column's last scale dword: a dword spans 4 row
      // blocks = two 64-row tiles; the even tile writes the odd one's bytes
      // as 0 when that tile does not exist, and a block past R is 0 as well
      uint8_t* cscale = p.col_codes ? p.col_scales + z * scale_bytes(p.C, p.R) + scale_offset(c, r / 32, p.C) : nullptr;
      if (cscale && r >= p.R) *cscale = 0;
      if (cscale && (blockIdx.y & 1) == 0 && r0 + kTileR >= p.R) cscale[2] = 0;
    }
    if (c < p.C && r < p.R) {
      float v[32];
      lds_col_block(tile, kPitch, blk * 32, col, v);
      if (p.partials) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) part = part + v[i];
        p.partials[z * (p.R / 32) * p.C + (r / 32) * p.C + c] = part;
      }
      if (p.col_codes) {
        uint8_t* codes = p.col_codes + z * p.C * (p.R * B / 8) + c * (p.R * B / 8) + r * B / 8;
        uint8_t* scales = p.col_scales + z * scale_bytes(p.C, p.R) + scale_offset(c, r / 32, p.C);
        quant_store<FMT, MODE, HAD>(v, codes, scales);
      }
    }
  }
}

// db[c] = sum over blocks b (increasing) of partials[b][c], from +0.
__global__ __launch_bounds__(256) void colsum_finish_kernel(const float* partials, int64_t nb, int64_t C,
                                                            float* out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t z = blockIdx.y;
  if (c >= C) return;
  const float* src = partials + z * nb * C;
  float s = 0.0f;
  for (int64_t b = 0; b < nb; ++b) s = s + src[b * C + c];
  out[z * C + c] = s;
}

using PackFn = void (*)(PackParams);

template <int FMT, int MODE, int HAD>
PackFn pick_pro(int pro) {
  switch (pro) {
    case kIdentity: return pack_kernel<FMT, MODE, HAD, kIdentity>;
    case kGelu: return pack_kernel<FMT, MODE, HAD, kGelu>;
    case kDGelu: return pack_kernel<FMT, MODE, HAD, kDGelu>;
    case kSwiglu: return pack_kernel<FMT, MODE, HAD, kSwiglu>;
    case kDSwiglu: return pack_kernel<FMT, MODE, HAD, kDSwiglu>;
    default: return nullptr;
  }
}

PackFn pick(int fmt, int mode, int had, int pro) {
  if (fmt == kE2M1 && mode == kFloor && !had) return pick_pro<kE2M1, kFloor, 0>(pro);
  if (fmt == kE2M3 && mode == kFloor && !had) return pick_pro<kE2M3, kFloor, 0>(pro);
  if (fmt == kE2M3 && mode == kFloor && had) return pick_pro<kE2M3, kFloor, 1>(pro);
  if (fmt == kE4M3 && mode == kRceil && !had) return pick_pro<kE4M3, kRceil, 0>(pro);
  if (fmt == kE4M3 && mode == kFloor && !had) return pick_pro<kE4M3, kFloor, 0>(pro);
  return nullptr;
}

}  // namespace

bool pack_supported(int fmt, int mode, int had, int pro) { return pick(fmt, mode, had, pro) != nullptr; }

hipError_t launch_pack(const PackParams& p, int fmt, int mode, int had, int pro, int64_t batch,
                       hipStream_t stream) {
  PackFn fn = pick(fmt, mode, had, pro);
  if (!fn) return hipErrorInvalidValue;
  dim3 grid((unsigned)((p.C + kTileC - 1) / kTileC), (unsigned)((p.R + kTileR - 1) / kTileR), (unsigned)batch);
  hipLaunchKernelGGL(fn, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_colsum_finish(const float* partials, int64_t nb, int64_t C, float* out, int64_t batch,
                                hipStream_t stream) {
  dim3 grid((unsigned)((C + 255) / 256), (unsigned)batch);
  hipLaunchKernelGGL(colsum_finish_kernel, grid, dim3(256), 0, stream, partials, nb, C, out);
  return hipGetLastError();
}

}  // namespace mx
