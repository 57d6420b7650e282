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
// Work split.  One 256-thread workgroup owns a 128-row x 128-column tile.
//  1. Load: each thread reads eight 16-byte chunks (8 bf16) -- a row of the
//     tile is 16 chunks, so a wavefront covers 4 rows x 256 B per load, fully
//     coalesced -- applies the prologue in registers, rounds to bf16 and
//     writes the tile to LDS.  The prologue output exists only on chip.
//  2. Row pass: threads quantize the 1x32 blocks (row q/4, block q%4).
//  3. Column pass: threads quantize the 32x1 blocks (column q/4, row block
//     q%4), written transposed as a K-major operand.
//     In both passes the four blocks a row or column has in the tile sit in
//     four adjacent lanes, so each store instruction writes 16 runs of 4
//     consecutive blocks plus 16 whole scale dwords.
// Rows/columns past R/C (multiples of 32) are masked per chunk.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

constexpr int kTileR = 128, kTileC = 128;
// bytes per LDS row: 256 B of data + 16 B pad; every 32-row block is
// shifted by a further 32 B so that the four row blocks of a column read
// in one column-pass instruction fall in different banks
constexpr int kPitch = kTileC * 2 + 16;
constexpr int kBlockSkew = 32;
constexpr int kTileBytes = kTileR * kPitch + 3 * kBlockSkew;
constexpr int kChunksPerRow = kTileC / 8;  // 16-byte chunks (8 bf16) per tile row
constexpr int kLoads = kTileR * kChunksPerRow / 256;  // chunks per thread
static_assert(256 / kChunksPerRow == 16 && kTileR == 16 * kLoads, "a load step is 16 tile rows");
__device__ __forceinline__ int lds_row(int row) { return row * kPitch + (row >> 5) * kBlockSkew; }

struct Chunk8 {
  uint32_t w[4];  // 8 bf16, element 2i in the low half of w[i]
};

// Raw input chunks of one tile position: up to three bf16 inputs.
template <int PRO>
struct Raw {
  static constexpr int kN = (PRO == kDGelu || PRO == kSwiglu) ? 2 : (PRO == kDSwiglu ? 3 : 1);
  uint4 in[kN];
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ Chunk8 as_chunk(const uint4 v) {
  Chunk8 c;
  c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  return c;
}

// Where the inputs behind logical chunk (r, c..c+7) start, and each input's
// row pitch in elements (the chunk of row r + d sits d pitches further on).
template <int PRO>
struct InputAt {
  const uint16_t* ptr[Raw<PRO>::kN];
  int64_t pitch[Raw<PRO>::kN];
};
template <int PRO>
__device__ __forceinline__ InputAt<PRO> input_at(const PackParams& p, const uint16_t* xb, const uint16_t* ab,
                                                 int64_t r, int64_t c) {
  InputAt<PRO> a;
  if constexpr (PRO == kIdentity || PRO == kGelu) {
    a.ptr[0] = xb + r * p.C + c;
    a.pitch[0] = p.C;
  } else if constexpr (PRO == kDGelu) {
    a.ptr[0] = xb + r * p.C + c;
    a.ptr[1] = ab + r * p.C + c;
    a.pitch[0] = a.pitch[1] = p.C;
  } else if constexpr (PRO == kSwiglu) {  // x = H [R][2C] = [gate | up]
    a.ptr[0] = xb + r * 2 * p.C + c;
    a.ptr[1] = xb + r * 2 * p.C + p.C + c;
    a.pitch[0] = a.pitch[1] = 2 * p.C;
  } else {  // kDSwiglu: C = 2F, x = dz [R][F], aux = H [R][2F]
    const int64_t F = p.C / 2;
    const int64_t j = c < F ? c : c - F;
    a.ptr[0] = xb + r * F + j;
    a.ptr[1] = ab + r * p.C + j;
    a.ptr[2] = ab + r * p.C + F + j;
    a.pitch[0] = F;
    a.pitch[1] = a.pitch[2] = p.C;
  }
  return a;
}

// Global loads of the inputs behind logical chunk (r, c..c+7).
template <int PRO>
__device__ __forceinline__ Raw<PRO> load_raw(const PackParams& p, const uint16_t* xb, const uint16_t* ab, int64_t r,
                                             int64_t c) {
  const InputAt<PRO> a = input_at<PRO>(p, xb, ab, r, c);
  Raw<PRO> q;
#pragma unroll
  for (int k = 0; k < Raw<PRO>::kN; ++k) q.in[k] = ld16(a.ptr[k]);
  return q;
}

// The prologue on one chunk, each result rounded to bf16 ([P1] commit
// messages: the activation epilogue becomes the packer's prologue).
template <int PRO>
__device__ __forceinline__ Chunk8 apply_prologue(const PackParams& p, const Raw<PRO>& q, int64_t c) {
  if constexpr (PRO == kIdentity) {
    return as_chunk(q.in[0]);
  } else {
    Chunk8 out;
    const Chunk8 x = as_chunk(q.in[0]);
    const Chunk8 y = as_chunk(q.in[Raw<PRO>::kN > 1 ? 1 : 0]);
    const Chunk8 u = as_chunk(q.in[Raw<PRO>::kN - 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo, hi;
      if constexpr (PRO == kGelu) {
        lo = gelu_bf16(bf16_lo(x.w[i]));
        hi = gelu_bf16(bf16_hi(x.w[i]));
      } else if constexpr (PRO == kDGelu) {
        lo = dgelu_bf16(bf16_lo(x.w[i]), bf16_lo(y.w[i]));
        hi = dgelu_bf16(bf16_hi(x.w[i]), bf16_hi(y.w[i]));
      } else if constexpr (PRO == kSwiglu) {
        lo = swiglu_bf16(bf16_lo(x.w[i]), bf16_lo(y.w[i]));
        hi = swiglu_bf16(bf16_hi(x.w[i]), bf16_hi(y.w[i]));
      } else {
        if (c < p.C / 2) {
          lo = dswiglu_gate_bf16(bf16_lo(x.w[i]), bf16_lo(y.w[i]), bf16_lo(u.w[i]));
          hi = dswiglu_gate_bf16(bf16_hi(x.w[i]), bf16_hi(y.w[i]), bf16_hi(u.w[i]));
        } else {
          lo = dswiglu_up_bf16(bf16_lo(x.w[i]), bf16_lo(y.w[i]));
          hi = dswiglu_up_bf16(bf16_hi(x.w[i]), bf16_hi(y.w[i]));
        }
      }
      // results are exact bf16 values
      out.w[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
    }
    return out;
  }
}

// ------------------------------------------------------------------ GELU table
// The GELU prologue's result is a function of one bf16 code, so a
// workgroup evaluates gelu_bf16 once per code of a window of magnitudes,
// [2^-16, 32) (exponent fields kLo .. kLo + kFields - 1), into an LDS table
// and looks the codes up: slot = (code & 0x7fff) - kA0 + (code >> 15) *
// kSlots.  Slot kN of each sign is a sentinel for codes outside the
// window (smaller, larger, infinite, NaN); a chunk holding one is
// recomputed from its inputs with gelu_bf16 after the lookups.  The other
// prologues keep their in-register arithmetic: their results also depend on
// the other inputs, and looking up only the one-code factor did not pay.
struct GeluTable {
  static constexpr uint32_t kLo = 111, kFields = 21;
  static constexpr uint32_t kA0 = kLo << 7, kN = kFields << 7, kSlots = kN + 1;
  static constexpr int kEntries = 2 * kSlots;
  static constexpr int kBytes = (kEntries * 2 + 15) & ~15;
  // workgroups per compute unit that the LDS allows (the kernel's launch
  // bounds hold its registers to that)
  static constexpr int kPerCU = (160 * 1024) / (kTileBytes + kBytes);
};
template <int PRO>
constexpr int kTableBytes = PRO == kGelu ? GeluTable::kBytes : 0;

// Fill the table (all 256 threads).
__device__ __forceinline__ void build_gelu_table(uint16_t* tab) {
  for (int i = threadIdx.x; i < GeluTable::kEntries; i += 256) {
    const uint32_t sgn = i >= (int)GeluTable::kSlots ? 1u : 0u;
    const uint32_t off = (uint32_t)i - sgn * GeluTable::kSlots;
    // the sentinel takes any code: its value is never used
    const uint32_t code = (sgn << 15) | (GeluTable::kA0 + (off < GeluTable::kN ? off : 0u));
    tab[i] = (uint16_t)(__float_as_uint(gelu_bf16(bf16_to_f32(code))) >> 16);
  }
}

// Slot of bf16 code `code` (low 16 bits); `out` gains 1 if it lies outside
// the window.
__device__ __forceinline__ uint32_t gelu_slot(uint32_t code, uint32_t& out) {
  uint32_t off = (code & 0x7fffu) - GeluTable::kA0;  // below the window wraps past kN
  off = off < GeluTable::kN ? off : GeluTable::kN;
  out |= (off == GeluTable::kN) ? 1u : 0u;
  return off + (code >> 15) * GeluTable::kSlots;
}

// GELU of one chunk by lookups; `out` gains 1 if a code lies outside the
// window.
__device__ __forceinline__ Chunk8 gelu_lookup(const uint4 in, const uint16_t* tab, uint32_t& out) {
  const Chunk8 x = as_chunk(in);
  Chunk8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = tab[gelu_slot(x.w[i] & 0xffffu, out)];
    const uint32_t hi = tab[gelu_slot(x.w[i] >> 16, out)];
    r.w[i] = lo | (hi << 16);
  }
  return r;
}

// One workgroup packs one 128 x 128 tile (column tile bx, row tile by) of
// batch entry z.
template <int FMT, int MODE, int HAD, int PRO, int SR = 0>
__device__ __forceinline__ void pack_tile(const PackParams& p, int64_t bx, int64_t by, int64_t z,
                                          uint8_t* tile) {
  static_assert(!SR || (FMT == kE2M1 && MODE == kFloor && !HAD), "stochastic rounding: MXFP4 only");
  constexpr int B = FmtTraits<FMT>::kBits;
  const int t = threadIdx.x;
  const int64_t r0 = by * kTileR, c0 = bx * kTileC;
  const int64_t in_cols = (PRO == kSwiglu) ? 2 * p.C : (PRO == kDSwiglu ? p.C / 2 : p.C);
  const uint16_t* xb = p.x + z * p.R * in_cols;
  const uint16_t* ab = p.aux ? p.aux + z * p.R * p.C : nullptr;

  // 1. load + prologue -> LDS (rows / columns past R / C are zero).  Load i
  //    of thread t reads chunk t % 16 of tile row t / 16 + 16 i: the column
  //    is the thread's own, the row steps by 16.
  Raw<PRO> raw[kLoads];
  const int row_t = t / kChunksPerRow, ch_t = t % kChunksPerRow;
  const int64_t c_t = c0 + ch_t * 8;
  // LDS offset of load i: lds_row(row_t + 16 i) + 16 ch_t, where the 32-row
  // block of row row_t + 16 i is i / 2 (row_t < 16)
  const int lds_t = row_t * kPitch + ch_t * 16;
  constexpr auto lds_step = [](int i) { return i * 16 * kPitch + (i >> 1) * kBlockSkew; };
  // GELU: the prologue by lookups in the table at tile + kTileBytes; bit i
  // of redo is set if chunk i holds a code outside the table window
  [[maybe_unused]] const uint16_t* gtab = reinterpret_cast<const uint16_t*>(tile + kTileBytes);
  [[maybe_unused]] uint32_t redo = 0;
  if (r0 + kTileR <= p.R && c0 + kTileC <= p.C) {
    // whole tile inside the tensor (uniform branch): one address per input,
    // stepped by 16 row pitches per load, and no masks
    const InputAt<PRO> a = input_at<PRO>(p, xb, ab, r0 + row_t, c_t);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
#pragma unroll
      for (int k = 0; k < Raw<PRO>::kN; ++k) raw[i].in[k] = ld16(a.ptr[k] + 16 * i * a.pitch[k]);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      Chunk8 v;
      if constexpr (PRO == kGelu) {
        uint32_t out = 0;
        v = gelu_lookup(raw[i].in[0], gtab, out);
        redo |= out << i;
      } else {
        v = apply_prologue<PRO>(p, raw[i], c_t);
      }
      *reinterpret_cast<uint4*>(tile + lds_t + lds_step(i)) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int64_t r = r0 + row_t + 16 * i;
      if (r < p.R && c_t < p.C) raw[i] = load_raw<PRO>(p, xb, ab, r, c_t);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int64_t r = r0 + row_t + 16 * i;
      Chunk8 v;
      if (r < p.R && c_t < p.C) {
        if constexpr (PRO == kGelu) {
          uint32_t out = 0;
          v = gelu_lookup(raw[i].in[0], gtab, out);
          redo |= out << i;
        } else {
          v = apply_prologue<PRO>(p, raw[i], c_t);
        }
      } else {
        v.w[0] = v.w[1] = v.w[2] = v.w[3] = 0u;
      }
      *reinterpret_cast<uint4*>(tile + lds_t + lds_step(i)) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
    }
  }
  if constexpr (PRO == kGelu) {
    // chunks with codes outside the window: every element again from its
    // input (rare for activations of ordinary magnitude)
    if (redo != 0) {
      const uint16_t* x = xb + (r0 + row_t) * p.C + c_t;
#pragma unroll 1
      for (int i = 0; i < kLoads; ++i) {
        if ((redo >> i) & 1u) {
          uint16_t* dst = reinterpret_cast<uint16_t*>(tile + lds_t + lds_step(i));
#pragma unroll 1
          for (int e = 0; e < 8; ++e)
            dst[e] = (uint16_t)(__float_as_uint(gelu_bf16(bf16_to_f32(x[16 * i * p.C + e]))) >> 16);
        }
      }
    }
  }
  __syncthreads();

  // 2. row pass: blocks (row q/4, blk q%4) along dim 1, q = t, t + 256; the
  //    four blocks of a row come from four adjacent lanes, so their codes and
  //    their scale dword are written as one contiguous run
  //    (the tile spans K group bx of its rows: scale_offset(r, 4 bx + blk, R)
  //    and code_group(r, c, R, B) are a tile base plus a small lane offset)
  if (p.row_codes) {
    uint8_t* const scale_base = p.row_scales + z * scale_bytes(p.R, p.C) + (bx * p.R + r0) * 4;
    uint8_t* const code_base = p.row_codes + z * code_bytes(p.R, p.C, B) + (bx * p.R + r0) * (16 * B);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = t + 256 * h;
      const int row = q >> 2, blk = q & 3;
      const int64_t r = r0 + row, c = c0 + blk * 32;
      if (r < p.R) {
        uint8_t* scales = scale_base + (row * 4 + blk);
        uint8_t* group = code_base + row * (16 * B);
        if (c < p.C) {
          float v[32];
          lds_row_block(tile + lds_row(row), 0, 0, blk * 32, v);
          if constexpr (SR)
            quant_store_sr(v, group, blk, r, scales, p.sr_seed, 0u, (uint64_t)((z * p.R + r) * p.C + c));
          else
            quant_store<FMT, MODE, HAD>(v, group, blk, r, scales);
        } else {
          // pad block of the row's last K group (a tile spans one group)
          *scales = 0;
          zero_block<FMT>(group, blk, r);
        }
      }
    }
  }

  // 3. column pass: blocks (column q/4, rows 32*(q%4) .. +31) along dim 0,
  //    q = t, t + 256; a column's four blocks come from four adjacent lanes
  //    (the tile spans K group by of its columns: scale_offset(c, 4 by + blk,
  //    C) and code_group(c, r, C, B) are a tile base plus a lane offset)
  if (p.col_codes || p.partials) {
    const int64_t scale_base = z * scale_bytes(p.C, p.R) + (by * p.C + c0) * 4;
    const int64_t code_base = z * code_bytes(p.C, p.R, B) + (by * p.C + c0) * (16 * B);
    float* const part_base = p.partials ? p.partials + z * (p.R / 32) * p.C + 4 * by * p.C + c0 : nullptr;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = t + 256 * h;
      const int col = q >> 2, blk = q & 3;
      const int64_t c = c0 + col, r = r0 + blk * 32;
      if (c < p.C) {
        if (r < p.R) {
          float v[32];
          const uint16_t* src = reinterpret_cast<const uint16_t*>(tile + lds_row(32 * blk)) + col;
#pragma unroll
          for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(src[i * (kPitch / 2)]);
          if (p.partials) {
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) part = part + v[i];
            part_base[blk * p.C + col] = part;
          }
          if (p.col_codes) {
            uint8_t* group = p.col_codes + code_base + col * (16 * B);
            uint8_t* scales = p.col_scales + scale_base + (col * 4 + blk);
            if constexpr (SR)
              quant_store_sr(v, group, blk, c, scales, p.sr_seed, 1u, (uint64_t)((z * p.C + c) * p.R + r));
            else
              quant_store<FMT, MODE, HAD>(v, group, blk, c, scales);
          }
        } else if (p.col_codes) {
          // a 128-row tile spans one K group; blocks past R are pad
          p.col_scales[scale_base + (col * 4 + blk)] = 0;
          zero_block<FMT>(p.col_codes + code_base + col * (16 * B), blk, c);
        }
      }
    }
  }
}

// GELU: each workgroup fills the table once, then packs tiles w,
// w + gridDim.x, ... (the launch gives it as many workgroups as fit at
// once); `at` maps a tile index to its (params, bx, by, z).
template <int FMT, int MODE, int HAD, class TileAt>
__device__ __forceinline__ void pack_gelu_tiles(uint32_t tiles, uint8_t* tile, const TileAt& at) {
  build_gelu_table(reinterpret_cast<uint16_t*>(tile + kTileBytes));
  __syncthreads();
  for (uint32_t w = blockIdx.x; w < tiles; w += gridDim.x) {
    at(w, [&](const PackParams& p, uint32_t bx, uint32_t by, uint32_t z) {
      pack_tile<FMT, MODE, HAD, kGelu>(p, bx, by, z, tile);
    });
    __syncthreads();  // the next tile's writes wait for this tile's column pass
  }
}

// Tile w of a tensor of tx column tiles and ty row tiles per batch entry:
// column tile fastest, then row tile, then batch entry.
template <class F>
__device__ __forceinline__ void tile_of(const PackParams& p, uint32_t w, F&& f) {
  const uint32_t tx = (uint32_t)((p.C + kTileC - 1) / kTileC), ty = (uint32_t)((p.R + kTileR - 1) / kTileR);
  const uint32_t row_tile = w / tx;
  f(p, w - row_tile * tx, row_tile % ty, row_tile / ty);
}

template <int FMT, int MODE, int HAD, int PRO, int SR = 0>
__global__ __launch_bounds__(256, PRO == kGelu ? GeluTable::kPerCU : 1) void pack_kernel(PackParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileBytes + kTableBytes<PRO>];
  if constexpr (PRO == kGelu) {
    const uint32_t tiles = (uint32_t)(((p.C + kTileC - 1) / kTileC) * ((p.R + kTileR - 1) / kTileR) * p.batch);
    pack_gelu_tiles<FMT, MODE, HAD>(tiles, tile, [&](uint32_t w, auto&& f) { tile_of(p, w, f); });
  } else {
    pack_tile<FMT, MODE, HAD, PRO, SR>(p, blockIdx.x, blockIdx.y, blockIdx.z, tile);
  }
}

// Several tensors in one launch: tile w of the launch is tile w - first[i]
// of item i, with first[i] <= w < first[i + 1]; an item's tiles are ordered
// column tile fastest, then row tile, then batch entry.  Workgroup w packs
// tile w (GELU: tiles w, w + gridDim.x, ...).
template <int FMT, int MODE, int HAD, int PRO>
__global__ __launch_bounds__(256, PRO == kGelu ? GeluTable::kPerCU : 1) void pack_many_kernel(PackMany m) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileBytes + kTableBytes<PRO>];
  if constexpr (PRO == kGelu) {
    pack_gelu_tiles<FMT, MODE, HAD>((uint32_t)m.first[m.n], tile, [&](uint32_t w, auto&& f) {
      int i = 0;
      while (i + 1 < m.n && w >= m.first[i + 1]) ++i;
      tile_of(m.p[i], (uint32_t)(w - m.first[i]), f);
    });
  } else {
    const int64_t w = blockIdx.x;
    int i = 0;
    while (i + 1 < m.n && w >= m.first[i + 1]) ++i;
    // tile counts of one launch fit 32 bits (the grid is one-dimensional)
    const uint32_t local = (uint32_t)(w - m.first[i]);
    const uint32_t tx = (uint32_t)((m.p[i].C + kTileC - 1) / kTileC), ty = (uint32_t)((m.p[i].R + kTileR - 1) / kTileR);
    const uint32_t row_tile = local / tx;
    pack_tile<FMT, MODE, HAD, PRO>(m.p[i], local - row_tile * tx, row_tile % ty, row_tile / ty, tile);
  }
}

// Workgroups of a GELU launch: as many as fit on the compute units at once,
// at most one per tile.
int64_t gelu_grid(int64_t tiles) {
  const int64_t slots = (int64_t)GeluTable::kPerCU * cu_count();
  return tiles < slots ? tiles : slots;
}

// db[c] = sum over blocks b (increasing) of partials[b][c], from +0.  One
// thread per column (64-thread workgroups, so that a few thousand columns
// still spread over the compute units).  The additions stay one sequential
// chain per column; the loads run ahead of it in batches of 32, the next
// batch in flight while the current one is added (a batch past the end
// re-loads the last one, so no load sits under a branch).
constexpr int kColsumThreads = 64;
__global__ __launch_bounds__(kColsumThreads) void colsum_finish_kernel(const float* partials, int64_t nb,
                                                                       int64_t C, float* out) {
  const int64_t c = (int64_t)blockIdx.x * kColsumThreads + threadIdx.x;
  const int64_t z = blockIdx.y;
  if (c >= C) return;
  const float* src = partials + z * nb * C + c;
  const int64_t full = nb / 32;  // whole batches
  float s = 0.0f;
  if (full > 0) {
    float cur[32], nxt[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) cur[i] = src[(int64_t)i * C];
    for (int64_t b = 0; b < full; ++b) {
      const int64_t nb0 = 32 * (b + 1 < full ? b + 1 : b);
#pragma unroll
      for (int i = 0; i < 32; ++i) nxt[i] = src[(nb0 + i) * C];
#pragma unroll
      for (int i = 0; i < 32; ++i) s = s + cur[i];
#pragma unroll
      for (int i = 0; i < 32; ++i) cur[i] = nxt[i];
    }
  }
  for (int64_t b = 32 * full; b < nb; ++b) s = s + src[b * C];
  out[z * C + c] = s;
}

using PackFn = void (*)(PackParams);
using PackManyFn = void (*)(PackMany);

// The kernel of one (format, scale mode, rotation, prologue) combination,
// for one tensor per launch (PackKernels) or several (ManyAsOne).
template <int FMT, int MODE, int HAD, int PRO>
struct PackKernels {
  static constexpr PackFn one = pack_kernel<FMT, MODE, HAD, PRO>;
};

template <template <int, int, int, int> class K, int FMT, int MODE, int HAD>
auto pick_pro(int pro) -> decltype(K<FMT, MODE, HAD, kIdentity>::one) {
  switch (pro) {
    case kIdentity: return K<FMT, MODE, HAD, kIdentity>::one;
    case kGelu: return K<FMT, MODE, HAD, kGelu>::one;
    case kDGelu: return K<FMT, MODE, HAD, kDGelu>::one;
    case kSwiglu: return K<FMT, MODE, HAD, kSwiglu>::one;
    case kDSwiglu: return K<FMT, MODE, HAD, kDSwiglu>::one;
    default: return nullptr;
  }
}

template <int FMT, int MODE, int HAD, int PRO>
struct ManyAsOne {
  static constexpr PackManyFn one = pack_many_kernel<FMT, MODE, HAD, PRO>;
};

// The served combinations (FLOOR for every format, RCEIL for E4M3, the
// rotation for E2M3), through kernel family K.
template <template <int, int, int, int> class K>
auto pick(int fmt, int mode, int had, int pro) -> decltype(K<kE2M1, kFloor, 0, kIdentity>::one) {
  if (fmt == kE2M1 && mode == kFloor && !had) return pick_pro<K, kE2M1, kFloor, 0>(pro);
  if (fmt == kE2M3 && mode == kFloor && !had) return pick_pro<K, kE2M3, kFloor, 0>(pro);
  if (fmt == kE2M3 && mode == kFloor && had) return pick_pro<K, kE2M3, kFloor, 1>(pro);
  if (fmt == kE4M3 && mode == kRceil && !had) return pick_pro<K, kE4M3, kRceil, 0>(pro);
  if (fmt == kE4M3 && mode == kFloor && !had) return pick_pro<K, kE4M3, kFloor, 0>(pro);
  return nullptr;
}

}  // namespace

bool pack_supported(int fmt, int mode, int had, int pro) { return pick<PackKernels>(fmt, mode, had, pro) != nullptr; }

hipError_t launch_pack(const PackParams& p, int fmt, int mode, int had, int pro, int64_t batch,
                       hipStream_t stream) {
  PackFn fn = pick<PackKernels>(fmt, mode, had, pro);
  if (!fn) return hipErrorInvalidValue;
  dim3 grid((unsigned)((p.C + kTileC - 1) / kTileC), (unsigned)((p.R + kTileR - 1) / kTileR), (unsigned)batch);
  if (pro == kGelu) {
    PackParams q = p;
    q.batch = batch;
    hipLaunchKernelGGL(fn, dim3((unsigned)gelu_grid((int64_t)grid.x * grid.y * grid.z)), dim3(256), 0, stream, q);
  } else {
    hipLaunchKernelGGL(fn, grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_pack_many(const PackMany& m, int fmt, int mode, int had, int pro, hipStream_t stream) {
  PackManyFn fn = pick<ManyAsOne>(fmt, mode, had, pro);
  if (!fn || m.n < 1 || m.n > kPackManyMax) return hipErrorInvalidValue;
  const int64_t tiles = m.first[m.n];
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3((unsigned)(pro == kGelu ? gelu_grid(tiles) : tiles)), dim3(256), 0, stream, m);
  return hipGetLastError();
}

hipError_t launch_pack_sr(const PackParams& p, int64_t batch, hipStream_t stream) {
  dim3 grid((unsigned)((p.C + kTileC - 1) / kTileC), (unsigned)((p.R + kTileR - 1) / kTileR), (unsigned)batch);
  hipLaunchKernelGGL((pack_kernel<kE2M1, kFloor, 0, kIdentity, 1>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_colsum_finish(const float* partials, int64_t nb, int64_t C, float* out, int64_t batch,
                                hipStream_t stream) {
  dim3 grid((unsigned)((C + kColsumThreads - 1) / kColsumThreads), (unsigned)batch);
  hipLaunchKernelGGL(colsum_finish_kernel, grid, dim3(kColsumThreads), 0, stream, partials, nb, C, out);
  return hipGetLastError();
}

}  // namespace mx
