// Block-scaled MX GEMM for gfx950: C = A . B^T on K-major packed operands,
// on the CDNA4 scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4: E8M0
// block scales applied inside the instruction, binary32 accumulation).
//
// [P1] "feat(mxfp6): MXFP6 (E2M3) Flux linears, a fused MLP, and the MLPerf
//      recipe": MXFP6 GEMMs for forward, dgrad and wgrad, bias added in the
//      store epilogue into the fp32 accumulator (description, commit
//      messages).
// [P3] "MXFP4 training for Flux models": MXFP4 GEMM, NT layout
//      (Troubleshooting); 256x256 tiles at the Flux QKV shape (Tuned GEMMs).
// [P4] "MXFP8 cudnn-fe Swiglu fused Grouped MLP fwd/bwd and wgrad group
//      gemm": ragged grouped GEMM with the expert picked from the tile
//      coordinate (expert sizes are 128-row multiples, so a tile never
//      spans two experts), SwiGLU / dSwiGLU epilogues that quantize rowwise 1x32 and
//      columnwise 32x1 in the same launch, ragged-K weight gradient writing
//      zeros for empty experts (commit messages).
//
// Tiling.  256 threads = 4 wavefronts in a 2 x 2 grid over a BM x BN output
// tile; a wavefront owns (BM/2) x (BN/2) = (BM/64) x (BN/64) MFMA tiles of
// 32 x 32, whose accumulators live in AGPRs (one wavefront per SIMD).
// 256 x 256 tiles instead run 512 threads = 8 wavefronts in a 2 x 4 grid
// (128 x 64 each, two per SIMD).  K
// advances BK elements per stage (128 for E2M1/E2M3, 64 for E4M3), in steps
// of 64 (one MFMA per output tile).  Stages form a ring of S = 3 or 4
// buffers in LDS filled by direct global -> LDS loads (global_load_lds:
// each lane's 16 bytes land at M0 + 16 * lane), so no registers are spent
// on staging.  A stage's rows are stored densely; the 16-byte chunks of each
// row are permuted (XOR for E2M1 / E4M3, a rotation for E2M3's six chunks)
// so that the 32 rows one operand read touches spread over all LDS banks.
// The main loop is software-pipelined by step: the LDS reads of the next
// step's operands, and the global loads of a stage S - 1 ahead, are threaded
// between the current step's MFMAs, and the one barrier per stage sits at
// the start of its last step, so that the next stage's first operands are
// read while the current stage's last MFMAs run.

// Dense tiles are ordered for cache reuse: workgroups are dealt round-robin
// to the 8 XCDs (each with its own L2), so consecutive workgroup ids are
// remapped to give every XCD a contiguous range of tiles, and each range is
// walked in groups of 8 tile rows so that concurrent tiles share A and B
// panels.
//
// MFMA operand layout (measured): lane l holds row l%32 of A (of B) and the
// 32-element K block g = l/32 of the 64-element step.  E2M1 / E2M3 take the
// block's 32 codes contiguously (16 / 24 bytes); E4M3 takes K [16g, 16g+16)
// in bytes 0-15 and [32+16g, 32+16g+16) in bytes 16-31.  The lane's scale
// operand is the E8M0 byte of (its row, block g).  The instruction computes
// X . Y^T with lane l's 16 accumulators holding rows 8*(i/4) + 4*(l/32) + i%4,
// column l%32; the kernel passes the B fragment as X and the A fragment as
// Y, so a lane holds C row l%32 and the four consecutive columns
// 8*(i/4) + 4*(l/32) + {0..3} for each i/4 -- 8 contiguous bytes of bf16.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <type_traits>

#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));


template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<kE4M3> { static constexpr int kCode = 0; };
template <> struct MfmaFmt<kE2M3> { static constexpr int kCode = 2; };
template <> struct MfmaFmt<kE2M1> { static constexpr int kCode = 4; };

// Threads per workgroup of a BM x BN tile: 8 wavefronts for 256 x 256 and
// for the SwiGLU / dSwiGLU epilogues' 128 x 256 (two per SIMD, so that the
// epilogue's long VALU dependency chains of one wavefront interleave with
// another's), else 4.
constexpr int tile_threads(int bm, int bn, int epi = 0) {
  return ((bm == 256 && bn == 256) || (bm == 128 && bn == 256 && (epi == 1 || epi == 2))) ? 512 : 256;
}

// OCC: workgroups resident per compute unit (1 or 2).  With 2, each takes at
// most half the LDS and, per wavefront, half the register file, so that one
// workgroup's MFMAs run while the other waits on its loads, its barrier or
// its prologue and epilogue.
template <int FMT, int BM, int BN, int MODE, int EPI, int OCC = 1>
struct Cfg {
  static_assert(OCC == 1 || OCC == 2, "workgroups per compute unit");
  static constexpr int kLds = 163840 / OCC;              // LDS bytes one workgroup may take
  static constexpr int kBits = FmtTraits<FMT>::kBits;
  // 256 x 256 tiles run 8 wavefronts (2 per SIMD, 2 x 4 over the tile, 128
  // accumulator registers each), so that one wavefront's MFMAs can cover
  // the other's LDS and barrier waits (measured 2-4% faster than 4
  // wavefronts of 256 accumulators each); the other shapes run 4 (2 x 2)
  static constexpr int kThreads = tile_threads(BM, BN, EPI);
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kWavesN = kWaves / 2;  // wavefronts across N (2 across M)
  // K elements per stage: one 128-element K group (64 / 96 / 128 bytes per
  // row); E4M3 tiles whose 128-element stages would not fit a ring of two in
  // the LDS, or whose accumulators take more than 144 registers (leaving too
  // few for double-buffered 8-register fragments), take half a group (64
  // bytes) per stage.  Every stage ends in a
  // workgroup barrier: at 256 x 256, two 128-element E4M3 stages measured
  // 4-8% faster than four of 64 (MXFP8 16384 x 9216 x 3072: 504 -> 466 us;
  // the grouped step 954 -> 899 us, same box).
  static constexpr int kAccRegs = (BM / 64) * (BN / kWavesN / 32) * 16;  // accumulator registers per lane
  static constexpr int kBK = FMT == kE4M3 && (2 * ((BM + BN) * 128 + 2048) > kLds || kAccRegs > 144) ? 64 : 128;
  static constexpr int kRowBytes = kBK * kBits / 8;      // 64 / 96 / 128 (or 64) bytes per row per stage
  static constexpr int kChunks = kRowBytes / 16;         // 16-byte chunks per row per stage
  static constexpr int kScaleDw = 1;                     // scale dword (4 blocks of 32 along K) per row per stage
  static constexpr int kSJ = 512 / kThreads;            // scale-dword loads per thread per stage (512 slots)
  // 16-byte loads per thread per stage; a tile side whose chunks do not fill
  // whole loads (192 rows of 96 bytes) leaves the last load of some
  // wavefronts idle: they load a valid chunk into a junk area, so that every
  // wavefront issues the same number of loads (the vmcnt waits count them)
  static constexpr int kAIters = (BM * kChunks + kThreads - 1) / kThreads;
  static constexpr int kBIters = (BN * kChunks + kThreads - 1) / kThreads;
  static constexpr int kARem = (BM * kChunks) % kThreads;  // slots of a partial last load (0: none)
  static constexpr int kBRem = (BN * kChunks) % kThreads;
  static_assert(kARem % 64 == 0 && kBRem % 64 == 0, "partial loads cover whole wavefronts");
  // The ring of kStages stage buffers is laid out region by region: the A
  // rows of buffers 0 .. S-1, then their B rows, then their scale dwords
  // ([A rows, then B rows], 512 slots), then a junk area for idle load
  // slots.  Every read of one operand from any buffer is then within the
  // 16-bit offset of a ds_read from one per-lane base.
  static constexpr int kARegion = BM * kRowBytes;
  static constexpr int kBRegion = BN * kRowBytes;
  static constexpr int kSRegion = kScaleDw * 512 * 4;
  static constexpr int kJunk = (kARem || kBRem) ? 1024 : 0;
  static constexpr int kStage = kARegion + kBRegion + kSRegion;  // bytes per stage
  static constexpr int kStages = (4 * kStage + kJunk <= kLds) ? 4 : (3 * kStage + kJunk <= kLds) ? 3 : 2;
  static_assert(kStages * kStage + kJunk <= kLds, "two stages fit the LDS");
  static constexpr int aoff(int b) { return b * kARegion; }
  static constexpr int boff(int b) { return kStages * kARegion + b * kBRegion; }
  static constexpr int soff(int b) { return kStages * (kARegion + kBRegion) + b * kSRegion; }
  static constexpr int kJOff = kStages * kStage;
  static constexpr int kWM = BM / 2, kWN = BN / kWavesN;
  static_assert(kWN % 32 == 0, "wavefront tile width");
  static constexpr int kMI = kWM / 32, kNJ = kWN / 32;
  static constexpr int kLoads = kAIters + kBIters + kSJ * kScaleDw;  // vector-memory instructions per stage per wave
  static_assert(BM + BN <= 512, "scale slots");
  // epilogue staging
  static constexpr int kCPitch = kWN * 2 + 8;         // bf16 store: per-wave kWM x kWN tile
  static constexpr int kZPitch = BN * 2 + 16;         // SwiGLU: gate | up tile BM x BN, then z in its gate half
  static constexpr int kDPitch = BN * 2 + 16;         // dSwiGLU: two BM x BN tiles, 16-byte rows
  static constexpr int kEpiBytes = EPI == kEpiSwiglu    ? BM * kZPitch
                                   : EPI == kEpiDSwiglu ? 2 * BM * kDPitch
                                                        : kWaves * kWM * kCPitch;
  static constexpr int kSmem = (kJOff + kJunk > kEpiBytes) ? kJOff + kJunk : kEpiBytes;
  static_assert(kSmem <= kLds, "LDS budget");
};

// Position of logical 16-byte chunk c of row r among the row's NCH stored
// chunks, chosen so that the 16-byte operand reads of one chunk by the 32
// rows of a wavefront (its two halves reading adjacent chunks) take the
// minimum four LDS cycles (measured with the bank-conflict counter on
// gfx950): NCH = 8 (128-byte rows): c ^ ((r ^ (r >> 3)) & 7);  NCH = 4
// (64-byte rows): c ^ ((r >> 2) & 3) -- a permutation that also depends on
// row bit 4, or on rows r >> 1, costs twice that;  NCH = 6 (96-byte rows,
// whose bases repeat every 8 rows modulo 64 banks): (c + ((r >> 3) & 1)) %
// 6, which moves rows 8..15 of every 16 by one 4-bank step.
template <int NCH>
__device__ __forceinline__ int chunk_pos(int r, int c) {
  static_assert(NCH == 4 || NCH == 6 || NCH == 8, "chunks per row");
  if constexpr (NCH == 6) { const int q = c + ((r >> 3) & 1); return q >= 6 ? q - 6 : q; }
  else if constexpr (NCH == 8) return c ^ ((r ^ (r >> 3)) & 7);
  else return c ^ ((r >> 2) & 3);
}
// Inverse: the logical chunk stored at position pos of row r.
template <int NCH>
__device__ __forceinline__ int chunk_at(int r, int pos) {
  if constexpr (NCH == 6) { const int q = pos - ((r >> 3) & 1); return q < 0 ? q + 6 : q; }
  else return chunk_pos<NCH>(r, pos);  // the XOR permutations are involutions
}

// The intrinsics below exist only for the GPU; their bodies are compiled in
// the device pass alone, so the host pass sees plain declarations.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
  // s_waitcnt: vmcnt[3:0] + vmcnt[5:4] at bits 15:14; expcnt (7) and lgkmcnt (15) left unconstrained
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
#endif
}

// Wait for every outstanding LDS read of this wavefront.
__device__ __forceinline__ void wait_lgkmcnt0() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt and expcnt unconstrained, lgkmcnt 0
#endif
}

// Workgroup barrier without a memory fence (the stage loads are awaited
// explicitly with vmcnt); the empty asm keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void stage_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#endif
}

// Direct global -> LDS copy of 16 (4) bytes per lane: lane l's bytes land at
// LDS byte address lds + 16 * l (lds + 4 * l); lds must be the same for the
// whole wavefront (it goes to M0, which an LDS DMA needs one wait state
// after writing).  Written as inline assembly: the compiler models the
// intrinsic as a flat access to both global memory and the LDS, and while
// one is in flight it turns every LDS wait it inserts into a wait for all
// outstanding reads.  Kernels order these loads with explicit vmcnt waits
// and barriers.
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
}
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
#endif
}
// The same from a wavefront-uniform base (scalar registers) plus a per-lane
// 32-bit byte offset, so that the per-lane part stays fixed across stages.
__device__ __forceinline__ void lds_dma16_s(const void* base, uint32_t off, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
#endif
}
__device__ __forceinline__ void lds_dma4_s(const void* base, uint32_t off, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
#endif
}

// A pointer the compiler must take as produced here: it stays in scalar
// registers (or is spilled) instead of being loaded again where it is used.
template <typename T>
__device__ __forceinline__ void held_in_sgprs(T*& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+s"(v));
#endif
}

// Materialize a kernel argument in scalar registers at this point.  The
// epilogue's arguments are pinned before the main loop: a scalar load still
// in flight there shares the LDS wait counter, and the compiler then turns
// every LDS wait in the loop into a wait for all outstanding reads.
template <typename T>
__device__ __forceinline__ void pin_arg(T v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"s"(v));
#endif
}

// Keep the machine scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
#endif
}

__device__ __forceinline__ int wave_uniform(int v) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_readfirstlane(v);
#else
  return v;
#endif
}

// Read one lane's A/B operand for K step ks of the stage from row r of the
// LDS tile (row base rowp); g = lane / 32 picks the 32-element K block.
template <int FMT, int NCH>
__device__ __forceinline__ v8i lds_operand(const uint8_t* rowp, int r, int ks, int g) {
  v8i v;
  if constexpr (FMT == kE4M3) {  // chunks 4 ks + g and 4 ks + 2 + g
    const v4i a = *reinterpret_cast<const v4i*>(rowp + 16 * chunk_pos<NCH>(r, 4 * ks + g));
    const v4i b = *reinterpret_cast<const v4i*>(rowp + 16 * chunk_pos<NCH>(r, 4 * ks + 2 + g));
    v = v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  } else if constexpr (FMT == kE2M1) {  // chunk 2 ks + g
    // the instruction reads 4 dwords of an E2M1 operand: the upper half is
    // left undefined so that those registers stay free
    const v4i a = *reinterpret_cast<const v4i*>(rowp + 16 * chunk_pos<NCH>(r, 2 * ks + g));
    v = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
  } else {
    // block b = 2 ks + g of the group: its first 16 bytes are chunk b, its
    // last 8 bytes half g (g ^ 1 in rows with bit 4 set) of chunk 4 + ks (the
    // E2M3 order inside a K group); the instruction reads 6 dwords of an
    // E2M3 operand.  Both reads are conflict-free across the 64 banks.
    const v4i w = *reinterpret_cast<const v4i*>(rowp + 16 * chunk_pos<NCH>(r, 2 * ks + g));
    const v2i h = *reinterpret_cast<const v2i*>(rowp + 16 * chunk_pos<NCH>(r, 4 + ks) + 8 * (g ^ ((r >> 4) & 1)));
    const v4i h4 = __builtin_shufflevector(h, h, 0, 1, -1, -1);
    v = __builtin_shufflevector(w, h4, 0, 1, 2, 3, 4, 5, -1, -1);
  }
  return v;
}

// Dense tile order: XCD-contiguous ranges, then groups of 8 tile rows.
__device__ __forceinline__ void dense_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  if ((T & 7) == 0) bid = (bid & 7) * (T >> 3) + (bid >> 3);
  const int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * GM;
  const int gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int r = bid - group * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

template <int FMT, int BM, int BN, int MODE, int EPI, int OCC = 1>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int bx, int by, int bz, uint8_t* smem) {
  using CF = Cfg<FMT, BM, BN, MODE, EPI, OCC>;
  constexpr int kBits = CF::kBits;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / CF::kWavesN, wn = wave % CF::kWavesN;
  constexpr int kThreads = CF::kThreads;
  const int lrow = lane & 31, g = lane >> 5;

  // ---------------------------------------------------------------- tile
  int tm, tn;
  int split = 0;  // split K: this workgroup's part of the K range
  if constexpr (MODE == kDense) {
    const int tiles_m = (int)(p.M / BM), tiles_n = (int)(p.N / BN);
    int local = bx;
    if constexpr (EPI == kEpiSplit) {  // workgroups [s * T, (s + 1) * T) compute part s
      split = bx / (tiles_m * tiles_n);
      local = bx - split * (tiles_m * tiles_n);
    }
    dense_tile(local, tiles_m, tiles_n, tm, tn);
  } else if constexpr (MODE == kRaggedM) {
    // 1-D grid of (row tile, column tile) pairs, column tiles fastest.  Each
    // XCD takes a contiguous range, so the tiles of one row panel (and of
    // one group's weights) share that XCD's L2 -- except under dSwiGLU,
    // whose epilogue reads H rows scattered over its tile and measured 17%
    // faster with consecutive tiles spread over the XCDs (the other
    // epilogues 3-7% slower that way).
    const int nt = (int)(EPI == kEpiSwiglu ? 2 * p.F / BN : p.N / BN);
    const int T = (int)gridDim.x;
    int bid = bx;
    if (EPI != kEpiDSwiglu && (T & 7) == 0) bid = (bid & 7) * (T >> 3) + (bid >> 3);
    tn = bid % nt;
    tm = bid / nt;
  } else {
    tn = bx;
    tm = by;
  }
  int64_t m0 = (int64_t)tm * BM;
  int64_t m_end = 0;  // ragged-M: end of this tile's group (rows of C it may write)
  const int64_t n0 = (int64_t)tn * BN;  // SwiGLU: tile tn covers z columns [tn*BN/2, (tn+1)*BN/2)
  int64_t kbeg = 0, kend = p.K;
  int64_t b_row0 = 0;  // first B row of this tile's group
  int64_t b_soff = 0;  // byte offset of this tile's group in the B scales (one blocked array per group)
  int64_t b_coff = 0;  // byte offset of this tile's group in the B codes (one K-group-major array per group)
  int64_t c_off = 0;   // element offset of this tile's group in C
  if constexpr (MODE == kRaggedM) {
    // Group gi's rows [start, end) are cut into ceil((end - start) / BM)
    // tiles (counts are multiples of 128, so a 256-row tile at a group's
    // end may hold 128 rows); row tile tm walks the groups in order.  Rows
    // of a tile past its group's end are loaded as the group's last row and
    // never stored, so nothing at or past the last end is read or written.
    // Offsets are a caller invariant; clamping them into [start, R] and down
    // to a multiple of 128 keeps every access inside the buffers (and every
    // 32-row column block inside one tile) even if they are broken.
    int64_t start = 0;
    int rem = tm, gi = -1;
    for (int q = 0; q < p.G; ++q) {
      int64_t e = p.offsets[q];
      e = (e < start ? start : (e > p.R ? p.R : e)) & ~(int64_t)127;
      const int64_t nt = (e - start + BM - 1) / BM;
      if (rem < nt) {
        gi = q;
        m0 = start + (int64_t)rem * BM;
        m_end = e;
        break;
      }
      rem -= (int)nt;
      start = e;
    }
    if (gi < 0) return;  // past the last group's tiles
    b_row0 = (int64_t)gi * p.b_group_rows;
    b_soff = (int64_t)gi * scale_bytes(p.b_group_rows, p.ktot);
    b_coff = (int64_t)gi * code_bytes(p.b_group_rows, p.ktot, kBits);
  }
  if constexpr (MODE == kDense && EPI == kEpiSplit) {
    {
      const int64_t part = p.K / p.split_k;
      kbeg = split * part;
      kend = kbeg + part;
      c_off = split * p.M * p.ldc;
    }
  }
  if constexpr (MODE == kRaggedK) {
    const int gi = bz;
    kbeg = gi ? p.offsets[gi - 1] : 0;
    kend = p.offsets[gi];
    kbeg = (kbeg < 0 ? 0 : (kbeg > p.R ? p.R : kbeg)) & ~(int64_t)127;
    kend = (kend < 0 ? 0 : (kend > p.R ? p.R : kend)) & ~(int64_t)127;
    if (kend < kbeg) kend = kbeg;
    c_off = (int64_t)gi * p.M * p.N;
  }
  // rows of the A / B operands (of one group's B): the stride between K
  // groups of their codes and scales
  const int64_t a_rows = p.M;
  const int64_t b_rows = MODE == kRaggedM ? p.b_group_rows : p.N;
  constexpr int kGB = 16 * kBits;  // code bytes of one row in one 128-element K group
  const int nk = (int)((kend - kbeg) / CF::kBK);

  // LDS row r of the B tile -> global B row
  auto b_row = [&](int r) -> int64_t {
    if constexpr (EPI == kEpiSwiglu) {
      const int64_t zb = (int64_t)tn * (BN / 2);
      return b_row0 + (r < BN / 2 ? zb + r : p.F + zb + (r - BN / 2));
    } else {
      return b_row0 + n0 + r;
    }
  };

  // ---------------------------------------------------------------- loads
  // Stage slot s (16-byte units, s = i * 256 + t for load i of thread t)
  // holds row s / kChunks, position s % kChunks, i.e. logical chunk
  // chunk_at(row, position) of the row's stage segment.  A stage lies inside
  // one 128-element K group: its segment of a row starts (k0 % 128) * bits/8
  // bytes into the row's kGB-byte run of that group.  Offsets from the
  // group's start are 32-bit (operands < 2 GiB).
  constexpr int BK = CF::kBK;
  uint32_t a_off[CF::kAIters], b_off[CF::kBIters];
#pragma unroll
  for (int i = 0; i < CF::kAIters; ++i) {
    const int q = t + kThreads * i, r = q / CF::kChunks, pos = q % CF::kChunks;
    const int rr = r < BM ? r : 0;  // junk slots read a valid chunk
    const int c = chunk_at<CF::kChunks>(rr, pos);
    const int64_t ar = MODE == kRaggedM && m0 + rr >= m_end ? m_end - 1 : m0 + rr;
    a_off[i] = (uint32_t)(ar * kGB + 16 * c);
  }
#pragma unroll
  for (int i = 0; i < CF::kBIters; ++i) {
    const int q = t + kThreads * i, r = q / CF::kChunks, pos = q % CF::kChunks;
    const int rr = r < BN ? r : 0;
    const int c = chunk_at<CF::kChunks>(rr, pos);
    b_off[i] = (uint32_t)(b_coff + (b_row(rr) - b_row0) * kGB + 16 * c);
  }
  // scale dwords (4 blocks of 32 along K, blocked layout): slot t + kThreads j
  // of [A rows | B rows]; slots past BM + BN load row 0's dword into unused
  // slots, so every wave issues the same number of loads.  BM and BN are
  // multiples of 64, so a wavefront's 64 slots are all A rows, all B rows or
  // all unused: each load takes a wavefront-uniform base and K-group stride
  // (scalar registers) and a fixed per-lane 32-bit offset, and no vector
  // address arithmetic is left in the main loop.
  static_assert(BM % 64 == 0 && BN % 64 == 0, "scale slots of a wavefront are one operand's");
  const uint8_t* s_base[CF::kSJ];
  uint32_t s_step[CF::kSJ];  // bytes between consecutive K groups
  uint32_t s_off[CF::kSJ];
#pragma unroll
  for (int j = 0; j < CF::kSJ; ++j) {
    const int r = t + kThreads * j;
    const int rw = wave_uniform(r);  // the wavefront's first slot
    const bool is_b = rw >= BM && rw < BM + BN;
    const int64_t ar = MODE == kRaggedM && m0 + (r < BM ? r : 0) >= m_end ? m_end - 1 : m0 + (r < BM ? r : 0);
    s_base[j] = is_b ? p.b_scales + b_soff : p.a_scales;
    s_off[j] = (uint32_t)(is_b ? (b_row(r - BM) - b_row0) * 4 : ar * 4);
    s_step[j] = (uint32_t)((is_b ? b_rows : a_rows) * 4);
  }
  // bytes between consecutive K groups of the A / B codes; every offset
  // into an operand fits 32 bits (operands < 2 GiB), so a stage's base is
  // one 32-bit product and one 64-bit add
  const uint32_t a_gb = (uint32_t)(a_rows * kGB), b_gb = (uint32_t)(b_rows * kGB);
  // the operand bases, held in scalar registers for the whole loop: taken
  // through an empty asm, the compiler cannot re-derive them by loading the
  // kernel argument again (a scalar load in the loop shares the LDS wait
  // counter, and its wait would also wait for every LDS read in flight)
  const uint8_t* a_codes = p.a_codes;
  const uint8_t* b_codes = p.b_codes;
  held_in_sgprs(a_codes);
  held_in_sgprs(b_codes);
  const int wave_u = wave_uniform(wave);
  const uint32_t smem_lds = wave_uniform((int)lds_addr(smem));  // LDS byte address of smem

  // Load q (0 <= q < kLoads) of stage k into ring buffer buf: A chunks, then
  // B chunks, then scale dwords (K group d, slot half j).  Every use sits in
  // fully unrolled code, so q is a constant and each use compiles to one
  // load instruction.
#define MX_PIECE(k, buf, q)                                                                               \
  do {                                                                                                   \
    const uint32_t k0_ = (uint32_t)kbeg + (uint32_t)(k) * BK;                                            \
    const uint32_t g_ = k0_ >> 7, w_ = (k0_ & 127) * kBits / 8;                                          \
    const uint32_t st_ = smem_lds;                                                                       \
    if ((q) < CF::kAIters) {                                                                             \
      const int i_ = (q) < CF::kAIters ? (q) : 0;                                                        \
      const bool junk_ = CF::kARem && i_ == CF::kAIters - 1 && wave_u * 64 >= CF::kARem;                 \
      lds_dma16_s(a_codes + (g_ * a_gb + w_), a_off[i_],                                                \
                  st_ + (junk_ ? CF::kJOff : CF::aoff(buf) + (i_ * kThreads + wave_u * 64) * 16));            \
    } else if ((q) < CF::kAIters + CF::kBIters) {                                                        \
      const int i_ = (q) >= CF::kAIters && (q) < CF::kAIters + CF::kBIters ? (q) - CF::kAIters : 0;      \
      const bool junk_ = CF::kBRem && i_ == CF::kBIters - 1 && wave_u * 64 >= CF::kBRem;                 \
      lds_dma16_s(b_codes + (g_ * b_gb + w_), b_off[i_],                                                \
                  st_ + (junk_ ? CF::kJOff : CF::boff(buf) + (i_ * kThreads + wave_u * 64) * 16));            \
    } else {                                                                                             \
      const int e_ = (q) >= CF::kAIters + CF::kBIters ? (q) - CF::kAIters - CF::kBIters : 0;             \
      const int d_ = e_ / CF::kSJ, j_ = e_ % CF::kSJ;                                                    \
      lds_dma4_s(s_base[j_] + (g_ + d_) * s_step[j_], s_off[j_],                                        \
               st_ + CF::soff(buf) + (d_ * 512 + j_ * kThreads + wave_u * 64) * 4);                     \
    }                                                                                                    \
  } while (0)
#define MX_ISSUE(k, buf)                                                                                  \
  do {                                                                                                   \
    _Pragma("unroll") for (int q_ = 0; q_ < CF::kLoads; ++q_) MX_PIECE(k, buf, q_);                     \
  } while (0)

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
  for (int i = 0; i < CF::kMI; ++i) arow[i] = wm * CF::kWM + 32 * i + lrow;
#pragma unroll
  for (int j = 0; j < CF::kNJ; ++j) {
    if constexpr (EPI == kEpiSwiglu) {  // j < NJ/2: gate columns, j >= NJ/2: the matching up columns
      constexpr int H = CF::kNJ / 2;
      brow[j] = (j < H ? 0 : BN / 2) + wn * (CF::kWN / 2) + 32 * (j % H) + lrow;
    } else {
      brow[j] = wn * CF::kWN + 32 * j + lrow;
    }
  }

  // Software pipeline over K steps of 64 (KS per stage).  The MFMAs of a step
  // use operand fragments already in registers; the LDS reads of the next
  // step's fragments are threaded between them, and so are the global -> LDS
  // loads of a stage S - 1 ahead.  Each A fragment is re-read right after
  // the last MFMA of the step that uses it; B fragments are double-buffered
  // by step parity for E2M1 / E2M3, and re-read after their last use like A
  // for E4M3, whose MFMAs take twice as long (the registers an E4M3 operand
  // needs do not fit twice).  The last step of stage it first waits for
  // stage it + 1 to land and passes the one barrier of the stage, so that
  // its MFMAs overlap the reads of stage it + 1's first fragments and
  // scales; after that barrier no wave reads buffer it % S any more, and the
  // loads of stage it + S may refill it.  The loads of a stage are issued
  // over a window of KS steps: the last step of stage st - S (after its
  // barrier), then the first KS - 1 steps of stage st - S + 1, so at every
  // barrier exactly the S - 2 stages after the awaited one may still be in
  // flight.  Stages past the last one re-load the last stage's K range into
  // their (free) ring buffers, and the last stage still passes its barrier
  // and reads "its successor", so the loop has no branches and every wait
  // count is a constant; the epilogue waits for those extra loads before it
  // reuses the LDS.
  constexpr int S = CF::kStages;
  constexpr int KS = BK / 64;
  constexpr bool kBDouble = KS == 2;
  constexpr int kMf = CF::kMI * CF::kNJ;  // MFMAs per step
  constexpr int kWin = KS * kMf;          // MFMA slots in a stage's load window
  constexpr int kPart0 = (CF::kLoads + KS - 1) / KS;  // loads in the window's first step
  static_assert(CF::kLoads <= 2 * kWin, "two loads per MFMA slot at most");
  static_assert(KS == 1 || KS == 2, "steps per stage");
  // fragment reads (and, across a stage boundary, the scale reads) go in
  // the first three quarters of a step's MFMA slots where the registers
  // allow, so that they have landed when the next step starts
  constexpr int kReadSlots = kMf > 4 ? (3 * kMf) / 4 : kMf;
  // slot of read unit u (issued after that slot's MFMA): spread over the
  // read slots, but a single-buffered fragment no earlier than the last MFMA
  // that uses it.  Units: [the scales,] A0, B0 .. B(NJ-1), A1 .. A(MI-1).
  auto read_slot = [](int u, bool with_scales) constexpr {
    const int nu = CF::kMI + CF::kNJ + (with_scales ? 1 : 0);
    const int v = with_scales ? u - 1 : u;
    const int nominal = u * kReadSlots / nu;
    int first = 0;
    if (v == 0 || v > CF::kNJ) first = (v == 0 ? 0 : v - CF::kNJ) * CF::kNJ + CF::kNJ - 1;  // A
    else if (v > 0 && !kBDouble) first = (CF::kMI - 1) * CF::kNJ + (v - 1);                 // B
    return nominal > first ? nominal : first;
  };

  v8i af[CF::kMI], bf[kBDouble ? 2 : 1][CF::kNJ];
  uint32_t sca[CF::kMI], scb[CF::kNJ];  // this stage's scale dwords, shifted so byte 0 is its block g
  uint32_t nsa[CF::kMI], nsb[CF::kNJ];  // the next stage's scale dwords as stored

  // scale dwords and operand fragments of ring buffer b (a constant)
  auto read_scales = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CF::kMI; ++i) nsa[i] = *reinterpret_cast<const uint32_t*>(smem + CF::soff(b) + arow[i] * 4);
#pragma unroll
    for (int j = 0; j < CF::kNJ; ++j)
      nsb[j] = *reinterpret_cast<const uint32_t*>(smem + CF::soff(b) + (BM + brow[j]) * 4);
  };
  // fragment v of a step (v = 0: A0, 1 .. NJ: B0 .. B(NJ-1), then A1 ..)
  auto read_frag = [&](int reg, int v, int b, int ks) __attribute__((always_inline)) {
    if (v == 0 || v > CF::kNJ) {
      const int i = v == 0 ? 0 : v - CF::kNJ;
      af[i] = lds_operand<FMT, CF::kChunks>(smem + CF::aoff(b) + arow[i] * CF::kRowBytes, arow[i], ks, g);
    } else {
      const int j = v - 1;
      bf[kBDouble ? reg : 0][j] =
          lds_operand<FMT, CF::kChunks>(smem + CF::boff(b) + brow[j] * CF::kRowBytes, brow[j], ks, g);
    }
  };

  // one step: stage it (in ring buffer B = it % S, a constant), K step ks
  auto step = [&](int it, auto ksc, auto bc) __attribute__((always_inline)) {
    constexpr int ks = decltype(ksc)::value, B = decltype(bc)::value;
    constexpr int cur = kBDouble ? ks : 0;  // B fragment buffer of this step
    constexpr int sel = 2 * ks;             // byte of the shifted scale dwords: block 2 ks + g of the stage
    constexpr bool last = ks == KS - 1;
    if (last) {
      wait_vmcnt<CF::kLoads * (S - 2)>();  // this wave's loads of stage it + 1 landed
      wait_lgkmcnt0();  // every read of buffer it % S done before the barrier frees it
      stage_barrier();
    }
    constexpr int rbuf = last ? (B + 1) % S : B;  // the next step's stage buffer
    constexpr int rks = last ? 0 : ks + 1;
    const int lst = last ? it + S : it + S - 1;  // stage whose loads this step issues
    constexpr int w = last ? 0 : ks + 1;         // ... and its window step
    const int lk = lst < nk ? lst : nk - 1;      // its K range (the last stage's past the end)
    constexpr int lbuf = last ? B : (B + S - 1) % S;
    constexpr int U = CF::kMI + CF::kNJ + (last ? 1 : 0);  // read units: [scales,] fragments
#pragma unroll
    for (int f = 0; f < kMf; ++f) {
      const int i = f / CF::kNJ, j = f % CF::kNJ;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          bf[cur][j], af[i], acc[i][j], MfmaFmt<FMT>::kCode, MfmaFmt<FMT>::kCode, sel, (int)scb[j], sel, (int)sca[i]);
      sched_fence();
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (read_slot(u, last) == f) {
          if (last && u == 0) read_scales(rbuf);
          else read_frag(cur ^ 1, last ? u - 1 : u, rbuf, rks);
        }
#pragma unroll
      for (int q = 0; q < CF::kLoads; ++q)
        if (q * kWin / CF::kLoads == w * kMf + f) MX_PIECE(lk, lbuf, q);
      sched_fence();
    }
  };
  auto stage = [&](int it, auto bc) __attribute__((always_inline)) {
    // K block of byte 0: g, or 2 (it & 1) + g for 64-element stages (a
    // dword holds the four blocks of one 128-element group)
    const int sh = 8 * g + (KS == 1 ? 16 * (it & 1) : 0);
#pragma unroll
    for (int i = 0; i < CF::kMI; ++i) sca[i] = nsa[i] >> sh;
#pragma unroll
    for (int j = 0; j < CF::kNJ; ++j) scb[j] = nsb[j] >> sh;
    step(it, std::integral_constant<int, 0>{}, bc);
    if constexpr (KS == 2) step(it, std::integral_constant<int, 1>{}, bc);
  };

  pin_arg(p.c);
  pin_arg(p.ldc);
  pin_arg(p.c_f32);
  if constexpr (EPI == kEpiStore || EPI == kEpiAccum || EPI == kEpiSplit) {
    pin_arg(p.bias);
    pin_arg(p.bias_f32);
  } else {
    pin_arg(p.F);
    pin_arg(p.R);
    pin_arg(p.q_mode);
    pin_arg(p.q_row_codes);
    pin_arg(p.q_row_scales);
    pin_arg(p.q_col_codes);
    pin_arg(p.q_col_scales);
    if constexpr (EPI == kEpiDSwiglu) pin_arg(p.aux);
  }
  if (nk > 0) {  // (a ragged-K group may be empty)
    // prologue: stages 0 .. S - 2 and the first window step of stage S - 1
    // in flight; stage 0's scales and first fragments read
#pragma unroll
    for (int st = 0; st < S - 1; ++st) MX_ISSUE(st < nk ? st : nk - 1, st);
#pragma unroll
    for (int q = 0; q < kPart0; ++q) MX_PIECE(S - 1 < nk ? S - 1 : nk - 1, S - 1, q);
    wait_vmcnt<CF::kLoads * (S - 2) + kPart0>();
    stage_barrier();
    read_scales(0);
#pragma unroll
    for (int v = 0; v < CF::kMI + CF::kNJ; ++v) read_frag(0, v, 0, 0);
    // unrolled by S so that every stage's ring buffer is a constant
    for (int it0 = 0; it0 < nk; it0 += S) {
      stage(it0, std::integral_constant<int, 0>{});
      if (it0 + 1 < nk) stage(it0 + 1, std::integral_constant<int, 1>{});
      if constexpr (S > 2) {
        if (it0 + 2 < nk) stage(it0 + 2, std::integral_constant<int, 2 % S>{});
      }
      if constexpr (S > 3) {
        if (it0 + 3 < nk) stage(it0 + 3, std::integral_constant<int, 3 % S>{});
      }
    }
    wait_vmcnt<0>();  // the loads past the last stage, before the LDS is reused
  }
#undef MX_PIECE
#undef MX_ISSUE
  __syncthreads();  // all wavefronts are done with the stage ring before the epilogue reuses LDS

  // ---------------------------------------------------------------- epilogues
  // Lane (row lrow, column group q = 8 * (e / 4) + 4 * g) of MFMA tile (i, j)
  // holds acc[i][j][4 * (e / 4) + 0..3] = C[row][col + 0..3].
  if constexpr (EPI == kEpiStore || EPI == kEpiAccum || EPI == kEpiSplit) {
    // bias of this lane's columns, read once (one uniform branch); a split
    // part is binary32 without the bias, which the reduction adds
    constexpr bool kPart = EPI == kEpiSplit;
    float bv[CF::kNJ][16];
    if (kPart || p.bias == nullptr) {
#pragma unroll
      for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) bv[j][e] = 0.0f;
    } else if (p.bias_f32) {
      const float* bias32 = reinterpret_cast<const float*>(p.bias);
#pragma unroll
      for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const float4 q = *reinterpret_cast<const float4*>(bias32 + n0 + wn * CF::kWN + 32 * j + 8 * e4 + 4 * g);
          bv[j][4 * e4 + 0] = q.x;
          bv[j][4 * e4 + 1] = q.y;
          bv[j][4 * e4 + 2] = q.z;
          bv[j][4 * e4 + 3] = q.w;
        }
    } else {
      const uint16_t* bias16 = reinterpret_cast<const uint16_t*>(p.bias);
#pragma unroll
      for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const uint2 q = *reinterpret_cast<const uint2*>(bias16 + n0 + wn * CF::kWN + 32 * j + 8 * e4 + 4 * g);
          bv[j][4 * e4 + 0] = bf16_lo(q.x);
          bv[j][4 * e4 + 1] = bf16_hi(q.x);
          bv[j][4 * e4 + 2] = bf16_lo(q.y);
          bv[j][4 * e4 + 3] = bf16_hi(q.y);
        }
    }
    // C += A . B^T (mx_gemm_accumulate: a weight gradient added into a
    // caller-owned main_grad): the previous C joins the binary32 result
    // after the bias, before the store's one rounding.  The old values of
    // one 32-row block of MFMA tiles are loaded together (no load sits under
    // a per-element branch); the accumulators themselves are never
    // rewritten.  A kernel of its own, so that the plain store's register
    // allocation is not touched.
    constexpr bool accumulate = EPI == kEpiAccum;
    auto load_old = [&](int i, float (&o)[CF::kNJ][16]) {
      const int64_t m = m0 + wm * CF::kWM + 32 * i + lrow;
      if (p.c_f32) {
        const float* Co = reinterpret_cast<const float*>(p.c) + m * p.ldc;
        float4 w[CF::kNJ][4];
#pragma unroll
        for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4)
            w[j][e4] = *reinterpret_cast<const float4*>(Co + n0 + wn * CF::kWN + 32 * j + 8 * e4 + 4 * g);
#pragma unroll
        for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            o[j][4 * e4 + 0] = w[j][e4].x;
            o[j][4 * e4 + 1] = w[j][e4].y;
            o[j][4 * e4 + 2] = w[j][e4].z;
            o[j][4 * e4 + 3] = w[j][e4].w;
          }
      } else {
        const uint16_t* Co = reinterpret_cast<const uint16_t*>(p.c) + m * p.ldc;
        uint2 w[CF::kNJ][4];
#pragma unroll
        for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4)
            w[j][e4] = *reinterpret_cast<const uint2*>(Co + n0 + wn * CF::kWN + 32 * j + 8 * e4 + 4 * g);
#pragma unroll
        for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            o[j][4 * e4 + 0] = bf16_lo(w[j][e4].x);
            o[j][4 * e4 + 1] = bf16_hi(w[j][e4].x);
            o[j][4 * e4 + 2] = bf16_lo(w[j][e4].y);
            o[j][4 * e4 + 3] = bf16_hi(w[j][e4].y);
          }
      }
    };
    // value of element e of MFMA tile (i, j): fl32(acc + bias) (+ old)
    if (kPart || p.c_f32) {
      float* C = reinterpret_cast<float*>(p.c) + c_off;
      auto store_f32 = [&](auto with_old) {
        constexpr bool kOld = decltype(with_old)::value;
#pragma unroll
        for (int i = 0; i < CF::kMI; ++i) {
          float o[CF::kNJ][16];
          if constexpr (kOld) load_old(i, o);
          const int64_t m = m0 + wm * CF::kWM + 32 * i + lrow;
          if (MODE == kRaggedM && m >= m_end) continue;
#pragma unroll
          for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int64_t n = n0 + wn * CF::kWN + 32 * j + 8 * e4 + 4 * g;
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                v[q] = acc[i][j][4 * e4 + q] + bv[j][4 * e4 + q];
                if constexpr (kOld) v[q] = v[q] + o[j][4 * e4 + q];
              }
              *reinterpret_cast<float4*>(C + m * p.ldc + n) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
      };
      if constexpr (accumulate) {
        store_f32(std::true_type{});
      } else {
#pragma unroll
        for (int i = 0; i < CF::kMI; ++i)
#pragma unroll
          for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int64_t m = m0 + wm * CF::kWM + 32 * i + lrow;
              const int64_t n = n0 + wn * CF::kWN + 32 * j + 8 * e4 + 4 * g;
              const v16f& a = acc[i][j];
              if (MODE == kRaggedM && m >= m_end) continue;
              *reinterpret_cast<float4*>(C + m * p.ldc + n) =
                  make_float4(a[4 * e4 + 0] + bv[j][4 * e4 + 0], a[4 * e4 + 1] + bv[j][4 * e4 + 1],
                              a[4 * e4 + 2] + bv[j][4 * e4 + 2], a[4 * e4 + 3] + bv[j][4 * e4 + 3]);
            }
      }
    } else {
      // bf16: stage the wavefront's tile in LDS with 8-byte writes, then
      // write 16-byte row chunks
      uint8_t* wt = smem + wave * CF::kWM * CF::kCPitch;
      auto stage_bf16 = [&](auto with_old) {
        constexpr bool kOld = decltype(with_old)::value;
#pragma unroll
        for (int i = 0; i < CF::kMI; ++i) {
          float o[CF::kNJ][16];
          if constexpr (kOld) load_old(i, o);
#pragma unroll
          for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int r = 32 * i + lrow, cl = 32 * j + 8 * e4 + 4 * g;
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                v[q] = acc[i][j][4 * e4 + q] + bv[j][4 * e4 + q];
                if constexpr (kOld) v[q] = v[q] + o[j][4 * e4 + q];
              }
              *reinterpret_cast<uint2*>(wt + r * CF::kCPitch + cl * 2) =
                  make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
      };
      // without a bias the sums are rounded as they are (one uniform branch)
      auto stage_sums = [&](auto with_bias) __attribute__((always_inline)) {
        constexpr bool kBias = decltype(with_bias)::value;
#pragma unroll
        for (int i = 0; i < CF::kMI; ++i)
#pragma unroll
          for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int r = 32 * i + lrow, cl = 32 * j + 8 * e4 + 4 * g;
              const v16f& a = acc[i][j];
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = kBias ? a[4 * e4 + q] + bv[j][4 * e4 + q] : a[4 * e4 + q];
              *reinterpret_cast<uint2*>(wt + r * CF::kCPitch + cl * 2) =
                  make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
      };
      if constexpr (accumulate) {
        stage_bf16(std::true_type{});
      } else if (p.bias != nullptr) {
        stage_sums(std::true_type{});
      } else {
        stage_sums(std::false_type{});
      }
      __syncthreads();
      uint16_t* C = reinterpret_cast<uint16_t*>(p.c) + c_off;
      constexpr int kRowChunks = CF::kWN / 8;
#pragma unroll 4
      for (int q = lane; q < CF::kWM * kRowChunks; q += 64) {
        const int r = q / kRowChunks, ch = q % kRowChunks;
        const uint2 lo = *reinterpret_cast<const uint2*>(wt + r * CF::kCPitch + ch * 16);
        const uint2 hi = *reinterpret_cast<const uint2*>(wt + r * CF::kCPitch + ch * 16 + 8);
        const int64_t m = m0 + wm * CF::kWM + r;
        if (MODE == kRaggedM && m >= m_end) continue;
        *reinterpret_cast<uint4*>(C + m * p.ldc + n0 + wn * CF::kWN + ch * 8) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
  } else if constexpr (EPI == kEpiSwiglu) {
    // A lane holds gate (j < NJ/2) and up (j + NJ/2) of the same (row, z
    // columns).  Both are staged in LDS as bf16, the gate half in columns
    // [0, BN/2) of the tile and the up half in [BN/2, BN).  Then each thread
    // takes 8-column chunks of z in row order: H's gate and up chunks go out
    // as coalesced 16-byte stores (a wavefront writes whole 256-byte row
    // segments of each half), and z = SwiGLU(gate, up) replaces the gate
    // chunk; z is then quantized rowwise and columnwise out of LDS.
    constexpr int H2 = CF::kNJ / 2;
    uint8_t* zt = smem;  // pitch kZPitch: the staged gate | up tile, then z in the gate half
    const int64_t zb = (int64_t)tn * (BN / 2);
    uint16_t* Hc = reinterpret_cast<uint16_t*>(p.c);
#pragma unroll
    for (int i = 0; i < CF::kMI; ++i)
#pragma unroll
      for (int j = 0; j < H2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int ml = wm * CF::kWM + 32 * i + lrow;
          const int zc = wn * (CF::kWN / 2) + 32 * j + 8 * e4 + 4 * g;
          const v16f& ag = acc[i][j];
          const v16f& au = acc[i][j + H2];
          *reinterpret_cast<uint2*>(zt + ml * CF::kZPitch + zc * 2) =
              make_uint2(pack_bf16x2(ag[4 * e4 + 0], ag[4 * e4 + 1]), pack_bf16x2(ag[4 * e4 + 2], ag[4 * e4 + 3]));
          *reinterpret_cast<uint2*>(zt + ml * CF::kZPitch + BN + zc * 2) =
              make_uint2(pack_bf16x2(au[4 * e4 + 0], au[4 * e4 + 1]), pack_bf16x2(au[4 * e4 + 2], au[4 * e4 + 3]));
        }
    __syncthreads();
    {
      constexpr int kChunksRow = BN / 16;                // 8-column chunks of z per tile row
      constexpr int kPer = BM * kChunksRow / kThreads;   // chunks per thread
      static_assert(BM * kChunksRow % kThreads == 0, "whole chunks per thread");
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int q = t + kThreads * k, row = q / kChunksRow, ch = q % kChunksRow;
        uint4* gp = reinterpret_cast<uint4*>(zt + row * CF::kZPitch + 16 * ch);
        const uint4 gw = *gp;
        const uint4 uw = *reinterpret_cast<const uint4*>(zt + row * CF::kZPitch + BN + 16 * ch);
        const int64_t m = m0 + row;
        if (m < m_end) {
          *reinterpret_cast<uint4*>(Hc + m * 2 * p.F + zb + 8 * ch) = gw;
          *reinterpret_cast<uint4*>(Hc + m * 2 * p.F + p.F + zb + 8 * ch) = uw;
        }
        const uint32_t gs[4] = {gw.x, gw.y, gw.z, gw.w}, us[4] = {uw.x, uw.y, uw.z, uw.w};
        uint32_t z[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
          z[w] = (__float_as_uint(swiglu_bf16(bf16_lo(gs[w]), bf16_lo(us[w]))) >> 16) |
                 (__float_as_uint(swiglu_bf16(bf16_hi(gs[w]), bf16_hi(us[w]))) & 0xffff0000u);
        *gp = make_uint4(z[0], z[1], z[2], z[3]);
      }
    }
    __syncthreads();
    constexpr int QB = FmtTraits<FMT>::kBits;
    constexpr int ZC = BN / 2;  // z columns in the tile
    for (int q = t; q < BM * (ZC / 32); q += kThreads) {
      const int row = q / (ZC / 32), blk = q % (ZC / 32);
      if (m0 + row >= m_end) continue;
      float v[32];
      lds_row_block(zt, CF::kZPitch, row, blk * 32, v);
      const int64_t m = m0 + row, col = zb + 32 * blk;
      if (p.q_mode == kRceil)
        quant_store<FMT, kRceil, 0>(v, p.q_row_codes + code_group(m, col, p.R, QB), (int)((col >> 5) & 3), m,
                                    p.q_row_scales + scale_offset(m, col / 32, p.R));
      else
        quant_store<FMT, kFloor, 0>(v, p.q_row_codes + code_group(m, col, p.R, QB), (int)((col >> 5) & 3), m,
                                    p.q_row_scales + scale_offset(m, col / 32, p.R));
    }
    for (int q = t; q < ZC * (BM / 32); q += kThreads) {
      const int col = q % ZC, rb2 = q / ZC;
      if (m0 + 32 * rb2 >= m_end) continue;
      float v[32];
      lds_col_block(zt, CF::kZPitch, rb2 * 32, col, v);
      const int64_t cz = zb + col, m = m0 + 32 * rb2;
      if (p.q_mode == kRceil)
        quant_store<FMT, kRceil, 0>(v, p.q_col_codes + code_group(cz, m, p.F, QB), (int)((m >> 5) & 3), cz,
                                    p.q_col_scales + scale_offset(cz, m / 32, p.F));
      else
        quant_store<FMT, kFloor, 0>(v, p.q_col_codes + code_group(cz, m, p.F, QB), (int)((m >> 5) & 3), cz,
                                    p.q_col_scales + scale_offset(cz, m / 32, p.F));
    }
  } else {  // kEpiDSwiglu
    // dz = bf16(acc) is staged in LDS tile tg first.  Then each thread takes
    // 8-column chunks of the tile in row order: H's gate and up chunks of
    // that row arrive as coalesced 16-byte loads (a wavefront reads whole
    // 512-byte row segments), dz comes from LDS, d_gate replaces dz in tg
    // and d_up goes to tile tu.  Both tiles are then quantized rowwise and
    // columnwise out of LDS.
    uint8_t* tg = smem;
    uint8_t* tu = smem + BM * CF::kDPitch;
    const uint16_t* H = p.aux;
#pragma unroll
    for (int i = 0; i < CF::kMI; ++i)
#pragma unroll
      for (int j = 0; j < CF::kNJ; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int ml = wm * CF::kWM + 32 * i + lrow;
          const int nl = wn * CF::kWN + 32 * j + 8 * e4 + 4 * g;
          const v16f& a = acc[i][j];
          *reinterpret_cast<uint2*>(tg + ml * CF::kDPitch + nl * 2) =
              make_uint2(pack_bf16x2(a[4 * e4 + 0], a[4 * e4 + 1]), pack_bf16x2(a[4 * e4 + 2], a[4 * e4 + 3]));
        }
    constexpr int kChunksRow = BN / 8;                    // 8-column chunks per tile row
    constexpr int kPer = BM * kChunksRow / kThreads;      // chunks per thread
    static_assert(BM * kChunksRow % kThreads == 0, "whole chunks per thread");
    // every H load of this thread in flight at once; rows past the group's
    // end (none while groups are 128-row multiples and BM = 128) read its
    // last row and are never stored
    uint4 hg[kPer], hu[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = t + kThreads * k, row = q / kChunksRow, ch = q % kChunksRow;
      const int64_t m = m0 + row;
      const uint16_t* hrow = H + (m < m_end ? m : m_end - 1) * 2 * p.F + n0 + 8 * ch;
      hg[k] = *reinterpret_cast<const uint4*>(hrow);
      hu[k] = *reinterpret_cast<const uint4*>(hrow + p.F);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = t + kThreads * k, row = q / kChunksRow, ch = q % kChunksRow;
      uint4* zp = reinterpret_cast<uint4*>(tg + row * CF::kDPitch + 16 * ch);
      const uint4 zw = *zp;
      const uint32_t zs[4] = {zw.x, zw.y, zw.z, zw.w};
      const uint32_t gs[4] = {hg[k].x, hg[k].y, hg[k].z, hg[k].w};
      const uint32_t us[4] = {hu[k].x, hu[k].y, hu[k].z, hu[k].w};
      uint32_t dg[4], du[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float g0, g1, u0, u1;
        dswiglu_pair_bf16(bf16_lo(zs[w]), bf16_lo(gs[w]), bf16_lo(us[w]), g0, u0);
        dswiglu_pair_bf16(bf16_hi(zs[w]), bf16_hi(gs[w]), bf16_hi(us[w]), g1, u1);
        dg[w] = (__float_as_uint(g0) >> 16) | (__float_as_uint(g1) & 0xffff0000u);
        du[w] = (__float_as_uint(u0) >> 16) | (__float_as_uint(u1) & 0xffff0000u);
      }
      const int64_t m = m0 + row;
      if (p.c && m < m_end)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.c) + m * p.F + n0 + 8 * ch) = zw;
      *zp = make_uint4(dg[0], dg[1], dg[2], dg[3]);
      *reinterpret_cast<uint4*>(tu + row * CF::kDPitch + 16 * ch) = make_uint4(du[0], du[1], du[2], du[3]);
    }
    __syncthreads();
    constexpr int QB = FmtTraits<FMT>::kBits;
    const int64_t W = 2 * p.F;  // dH width
    for (int q = t; q < 2 * BM * (BN / 32); q += kThreads) {
      const int half = q / (BM * (BN / 32)), rq = q % (BM * (BN / 32));
      const int row = rq / (BN / 32), blk = rq % (BN / 32);
      if (m0 + row >= m_end) continue;
      float v[32];
      lds_row_block(half ? tu : tg, CF::kDPitch, row, blk * 32, v);
      const int64_t m = m0 + row, col = (half ? p.F : 0) + n0 + 32 * blk;
      if (p.q_mode == kRceil)
        quant_store<FMT, kRceil, 0>(v, p.q_row_codes + code_group(m, col, p.R, QB), (int)((col >> 5) & 3), m,
                                    p.q_row_scales + scale_offset(m, col / 32, p.R));
      else
        quant_store<FMT, kFloor, 0>(v, p.q_row_codes + code_group(m, col, p.R, QB), (int)((col >> 5) & 3), m,
                                    p.q_row_scales + scale_offset(m, col / 32, p.R));
    }
    for (int q = t; q < 2 * BN * (BM / 32); q += kThreads) {
      const int half = q / (BN * (BM / 32)), cq = q % (BN * (BM / 32));
      const int col = cq % BN, rb2 = cq / BN;
      if (m0 + 32 * rb2 >= m_end) continue;
      float v[32];
      lds_col_block(half ? tu : tg, CF::kDPitch, rb2 * 32, col, v);
      const int64_t cw = (half ? p.F : 0) + n0 + col, m = m0 + 32 * rb2;
      if (p.q_mode == kRceil)
        quant_store<FMT, kRceil, 0>(v, p.q_col_codes + code_group(cw, m, W, QB), (int)((m >> 5) & 3), cw,
                                    p.q_col_scales + scale_offset(cw, m / 32, W));
      else
        quant_store<FMT, kFloor, 0>(v, p.q_col_codes + code_group(cw, m, W, QB), (int)((m >> 5) & 3), cw,
                                    p.q_col_scales + scale_offset(cw, m / 32, W));
    }
  }
}

// One launch, one GEMM (or one grouped GEMM): workgroup (x, y, z) computes
// tile (x, y) of group z.
template <int FMT, int BM, int BN, int MODE, int EPI, int OCC = 1>
__global__ __launch_bounds__(tile_threads(BM, BN, EPI), OCC) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg<FMT, BM, BN, MODE, EPI, OCC>::kSmem];
  gemm_tile<FMT, BM, BN, MODE, EPI, OCC>(p, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

// The dense tile shapes {BM, BN, workgroups per compute unit}, in the order
// of GemmMany::shape.
constexpr int kNumDense = 8;
constexpr int kDenseShapes[kNumDense][3] = {{256, 256, 1}, {256, 192, 1}, {192, 256, 1}, {192, 192, 1},
                                            {256, 128, 1}, {256, 128, 2}, {128, 256, 2}, {192, 192, 2}};

template <int FMT, int SH>
using DenseCfg = Cfg<FMT, kDenseShapes[SH][0], kDenseShapes[SH][1], kDense, kEpiStore, kDenseShapes[SH][2]>;

template <int FMT, int SH>
__device__ __forceinline__ void dense_tile_sh(const GemmParams& p, int local, uint8_t* smem) {
  gemm_tile<FMT, kDenseShapes[SH][0], kDenseShapes[SH][1], kDense, kEpiStore, kDenseShapes[SH][2]>(p, local, 0, 0,
                                                                                                    smem);
}

// Several dense GEMMs in one launch: workgroup w computes tile
// w - first[i] of GEMM i (first[i] <= w < first[i + 1]) with that GEMM's
// tile shape, SA or SB (indices into kDenseShapes); the branch is uniform
// across the workgroup.  Both shapes run the same number of wavefronts.
template <int FMT, int SA, int SB>
__global__ __launch_bounds__(tile_threads(kDenseShapes[SA][0], kDenseShapes[SA][1]), kDenseShapes[SA][2]) void gemm_many_kernel(GemmMany m) {
  static_assert(DenseCfg<FMT, SA>::kThreads == DenseCfg<FMT, SB>::kThreads, "one workgroup size per launch");
  static_assert(kDenseShapes[SA][2] == kDenseShapes[SB][2], "one residency per launch");
  constexpr int kA = DenseCfg<FMT, SA>::kSmem, kB = DenseCfg<FMT, SB>::kSmem;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kA > kB ? kA : kB];
  const int w = blockIdx.x;
  int i = 0;
  while (i + 1 < m.n && w >= m.first[i + 1]) ++i;
  const int local = w - m.first[i];
  if (SA == SB || m.shape[i] == SA) dense_tile_sh<FMT, SA>(m.p[i], local, smem);
  else dense_tile_sh<FMT, SB>(m.p[i], local, smem);
}

template <int FMT, int BM, int BN, int MODE, int EPI, int OCC = 1>
hipError_t launch_one(const GemmParams& p, hipStream_t stream) {
  dim3 grid;
  if (MODE == kDense) {
    const int64_t parts = EPI == kEpiSplit ? p.split_k : 1;
    if (parts < 1) return hipErrorInvalidValue;
    if ((p.M / BM) * (p.N / BN) * parts >= (1ll << 31)) return hipErrorInvalidValue;
    grid = dim3((unsigned)((p.M / BM) * (p.N / BN) * parts), 1, 1);
  } else if (MODE == kRaggedM) {
    // column tiles x an upper bound on the row tiles: sum over groups of
    // ceil(count / BM) <= R / BM + G; the surplus workgroups exit at once
    const int64_t nt = EPI == kEpiSwiglu ? 2 * p.F / BN : p.N / BN;
    const int64_t rows = p.R > 0 ? (p.R + BM - 1) / BM + p.G : 0;
    if (nt * rows >= (1ll << 31)) return hipErrorInvalidValue;
    grid = dim3((unsigned)(nt * rows), 1, 1);
  } else {
    grid = dim3((unsigned)(p.N / BN), (unsigned)(p.M / BM), (unsigned)p.G);
  }
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<FMT, BM, BN, MODE, EPI, OCC>), grid, dim3(Cfg<FMT, BM, BN, MODE, EPI, OCC>::kThreads),
                     0, stream, p);
  return hipGetLastError();
}

// Dense tile shape (index into kDenseShapes): the one whose rounds of one
// tile per compute unit cost the least output area (rounds x BM x BN),
// larger tiles first on ties -- e.g. 4096 x 3072 takes 256 tiles of
// 256 x 192 in one round instead of 192 tiles of 256 x 256 on 192 of the 256
// compute units.  -1: no shape divides M x N.
int dense_shape(int64_t M, int64_t N) {
  const int64_t cus = cu_count();
  int best = -1;
  int64_t best_cost = 0;
  for (int i = 0; i < kNumDense; ++i) {
    const int bm = kDenseShapes[i][0], bn = kDenseShapes[i][1];
    if (kDenseShapes[i][2] != 1 || M % bm || N % bn) continue;
    const int64_t tiles = (M / bm) * (N / bn);
    const int64_t cost = ((tiles + cus - 1) / cus) * bm * bn;
    if (best < 0 || cost < best_cost) {
      best = i;
      best_cost = cost;
    }
  }
  return best;
}

// Measured launch plans (tile, workgroups per CU, K split) for the shapes
// of the Flux-12B block linears where the best of a sweep over every dense
// tiling and K split beat the rounds x tile-area rule: compute units,
// format, M, N, K, then the plan.  A plan with split_k > 1 needs a
// workspace, so mx_gemm (which has none) takes the rule for those shapes.
struct Tuned {
  int cus, fmt;
  int64_t M, N, K;
  GemmPlan plan;
};
constexpr Tuned kTuned[] = {
#include "mx_tuned.inc"
    {0, 0, 0, 0, 0, {0, 0, 0, 0}},  // end (no device has 0 compute units)
};

const Tuned* tuned(int fmt, int64_t M, int64_t N, int64_t K) {
  const int cus = cu_count();
  for (const Tuned& t : kTuned)
    if (t.cus == cus && t.fmt == fmt && t.M == M && t.N == N && t.K == K) return &t;
  return nullptr;
}

int shape_index(int bm, int bn, int wg) {
  for (int i = 0; i < kNumDense; ++i)
    if (kDenseShapes[i][0] == bm && kDenseShapes[i][1] == bn && kDenseShapes[i][2] == wg) return i;
  return -1;
}

// The shape a dense launch uses: the caller's (p.tile_shape = 1 + its
// index), else a tuned plan's without a K split, else the one dense_shape
// picks.
int dense_shape_of(int fmt, const GemmParams& p) {
  if (p.tile_shape > 0 && p.tile_shape <= kNumDense) return p.tile_shape - 1;
  const Tuned* t = tuned(fmt, p.M, p.N, p.K);
  if (t && t->plan.split_k <= 1) {
    const int i = shape_index(t->plan.tile_m, t->plan.tile_n, t->plan.wg_per_cu);
    if (i >= 0 && p.M % kDenseShapes[i][0] == 0 && p.N % kDenseShapes[i][1] == 0) return i;
  }
  return dense_shape(p.M, p.N);
}

// Split-K reduction: thread q sums 4 consecutive columns of one row over the
// parts in order, adds the bias and rounds once.
template <int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int64_t M, int64_t N,
                                                            const void* __restrict__ bias, int bias_f32,
                                                            void* __restrict__ c, int c_f32, int64_t ldc) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n4 = N / 4;
  if (q >= M * n4) return;
  const int64_t m = q / n4, n = (q - m * n4) * 4;
  const float* src = ws + m * N + n;
  float4 v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) v[s] = *reinterpret_cast<const float4*>(src + s * (M * N));
  float4 a = v[0];
#pragma unroll
  for (int s = 1; s < S; ++s) {
    a.x = a.x + v[s].x;
    a.y = a.y + v[s].y;
    a.z = a.z + v[s].z;
    a.w = a.w + v[s].w;
  }
  if (bias != nullptr) {
    float4 b;
    if (bias_f32) {
      b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(bias) + n);
    } else {
      const uint2 h = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(bias) + n);
      b = make_float4(bf16_lo(h.x), bf16_hi(h.x), bf16_lo(h.y), bf16_hi(h.y));
    }
    a.x = a.x + b.x;
    a.y = a.y + b.y;
    a.z = a.z + b.z;
    a.w = a.w + b.w;
  }
  if (c_f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + m * ldc + n) = a;
  } else {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(c) + m * ldc + n) =
        make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
  }
}

template <int FMT, int EPI>
hipError_t launch_dense(const GemmParams& p, hipStream_t stream) {
  switch (dense_shape_of(FMT, p)) {
    case 0: return launch_one<FMT, 256, 256, kDense, EPI>(p, stream);
    case 1: return launch_one<FMT, 256, 192, kDense, EPI>(p, stream);
    case 2: return launch_one<FMT, 192, 256, kDense, EPI>(p, stream);
    case 3: return launch_one<FMT, 192, 192, kDense, EPI>(p, stream);
    case 4: return launch_one<FMT, 256, 128, kDense, EPI>(p, stream);
    case 5: return launch_one<FMT, 256, 128, kDense, EPI, 2>(p, stream);
    case 6: return launch_one<FMT, 128, 256, kDense, EPI, 2>(p, stream);
    case 7: return launch_one<FMT, 192, 192, kDense, EPI, 2>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT>
hipError_t launch_fmt(const GemmParams& p, int mode, int epi, hipStream_t stream) {
  if (mode == kDense) {
    if (epi == kEpiAccum) return launch_dense<FMT, kEpiAccum>(p, stream);
    if (epi == kEpiSplit) return launch_dense<FMT, kEpiSplit>(p, stream);
    return launch_dense<FMT, kEpiStore>(p, stream);
  }
  if (mode == kRaggedM) {
    // 256-row tiles for the plain store.  The epilogues that quantize take
    // 128 rows with 8 wavefronts: dSwiGLU's two bf16 LDS tiles would not fit
    // at 256, and SwiGLU measured 8-9% faster (at expert sizes that are
    // multiples of 128, every 128-row tile is full, so no round ends part
    // empty; the plain store gained nothing from it)
    if (epi == kEpiSwiglu) return launch_one<FMT, 128, 256, kRaggedM, kEpiSwiglu>(p, stream);
    if (epi == kEpiDSwiglu) return launch_one<FMT, 128, 256, kRaggedM, kEpiDSwiglu>(p, stream);
    return launch_one<FMT, 256, 256, kRaggedM, kEpiStore>(p, stream);
  }
  return launch_one<FMT, 256, 256, kRaggedK, kEpiStore>(p, stream);
}

// Workgroup ranges of a many-launch whose shapes are set.
bool plan_many(GemmMany& m) {
  int64_t tiles = 0;
  for (int i = 0; i < m.n; ++i) {
    const int sh = m.shape[i];
    m.first[i] = (int)tiles;
    tiles += (m.p[i].M / kDenseShapes[sh][0]) * (m.p[i].N / kDenseShapes[sh][1]);
  }
  m.first[m.n] = (int)tiles;
  return tiles < (1ll << 31);
}

template <int FMT, int SA, int SB>
hipError_t launch_many_k(GemmMany m, hipStream_t stream) {
  if (!plan_many(m)) return hipErrorInvalidValue;
  const unsigned tiles = (unsigned)m.first[m.n];
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_many_kernel<FMT, SA, SB>), dim3(tiles), dim3(DenseCfg<FMT, SA>::kThreads), 0, stream, m);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_many_single(const GemmMany& m, int sh, hipStream_t stream) {
  switch (sh) {
    case 0: return launch_many_k<FMT, 0, 0>(m, stream);
    case 1: return launch_many_k<FMT, 1, 1>(m, stream);
    case 2: return launch_many_k<FMT, 2, 2>(m, stream);
    case 3: return launch_many_k<FMT, 3, 3>(m, stream);
    case 4: return launch_many_k<FMT, 4, 4>(m, stream);
    case 5: return launch_many_k<FMT, 5, 5>(m, stream);
    case 6: return launch_many_k<FMT, 6, 6>(m, stream);
    case 7: return launch_many_k<FMT, 7, 7>(m, stream);
    default: return hipErrorInvalidValue;
  }
}

// Two tile shapes can share a launch when they run the same number of
// wavefronts at the same residency: the 4-wavefront shapes at one workgroup
// per CU (256x192, 192x256, 192x192, 256x128) pairwise, and those at two
// (256x128, 128x256, 192x192) pairwise except 128x256 with 192x192 (their
// union spills at half the register file).  256x256 runs 8 wavefronts
// alone.
constexpr bool pairable(int a, int b) {
  return a != b && a != 0 && b != 0 && kDenseShapes[a][2] == kDenseShapes[b][2] && !(a == 6 && b == 7) &&
         !(a == 7 && b == 6);
}
template <int FMT>
hipError_t launch_many_pair(const GemmMany& m, int a, int b, hipStream_t stream) {
  switch (a * kNumDense + b) {  // a < b
    case 1 * kNumDense + 2: return launch_many_k<FMT, 1, 2>(m, stream);
    case 1 * kNumDense + 3: return launch_many_k<FMT, 1, 3>(m, stream);
    case 1 * kNumDense + 4: return launch_many_k<FMT, 1, 4>(m, stream);
    case 2 * kNumDense + 3: return launch_many_k<FMT, 2, 3>(m, stream);
    case 2 * kNumDense + 4: return launch_many_k<FMT, 2, 4>(m, stream);
    case 3 * kNumDense + 4: return launch_many_k<FMT, 3, 4>(m, stream);
    case 5 * kNumDense + 6: return launch_many_k<FMT, 5, 6>(m, stream);
    case 5 * kNumDense + 7: return launch_many_k<FMT, 5, 7>(m, stream);
    default: return hipErrorInvalidValue;
  }
}

// The GEMMs grouped into launches: the shapes in use taken in table order,
// each with the first later shape it can share a launch with (a linear
// layer's forward / data-gradient 256x192 and weight-gradient 192x192 at
// the Flux shapes are one such pair); items keep their order in a launch.
template <int FMT>
hipError_t launch_many_fmt(const GemmMany& all, hipStream_t stream) {
  bool used[kNumDense] = {};
  for (int i = 0; i < all.n; ++i) used[all.shape[i]] = true;
  for (int a = 0; a < kNumDense; ++a) {
    if (!used[a]) continue;
    used[a] = false;
    int b = -1;
    for (int k = a + 1; k < kNumDense && b < 0; ++k)
      if (used[k] && pairable(a, k)) b = k;
    if (b >= 0) used[b] = false;
    GemmMany m;
    memset(&m, 0, sizeof m);
    for (int i = 0; i < all.n; ++i)
      if (all.shape[i] == a || all.shape[i] == b) {
        m.p[m.n] = all.p[i];
        m.shape[m.n] = all.shape[i];
        ++m.n;
      }
    const hipError_t e = b >= 0 ? launch_many_pair<FMT>(m, a, b, stream) : launch_many_single<FMT>(m, a, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int dense_tile_index(int bm, int bn, int wg_per_cu, int64_t M, int64_t N) {
  for (int i = 0; i < kNumDense; ++i)
    if (kDenseShapes[i][0] == bm && kDenseShapes[i][1] == bn && kDenseShapes[i][2] == wg_per_cu)
      return (M % bm || N % bn) ? -1 : i;
  return -1;
}

hipError_t launch_gemm_many(GemmMany m, int fmt, hipStream_t stream) {
  if (m.n < 1 || m.n > kGemmManyMax) return hipErrorInvalidValue;
  for (int i = 0; i < m.n; ++i)
    if ((m.shape[i] = dense_shape_of(fmt, m.p[i])) < 0) return hipErrorInvalidValue;
  switch (fmt) {
    case kE2M1: return launch_many_fmt<kE2M1>(m, stream);
    case kE2M3: return launch_many_fmt<kE2M3>(m, stream);
    case kE4M3: return launch_many_fmt<kE4M3>(m, stream);
    default: return hipErrorInvalidValue;
  }
}

bool plan_gemm(int fmt, int64_t M, int64_t N, int64_t K, GemmPlan* out) {
  if (const Tuned* t = tuned(fmt, M, N, K)) {
    *out = t->plan;
    return true;
  }
  const int sh = dense_shape(M, N);
  if (sh < 0) return false;
  *out = GemmPlan{kDenseShapes[sh][0], kDenseShapes[sh][1], kDenseShapes[sh][2], 1};
  return true;
}

hipError_t launch_splitk_reduce(const float* ws, int split_k, int64_t M, int64_t N, const void* bias, int bias_f32,
                                void* c, int c_f32, int64_t ldc, hipStream_t stream) {
  const int64_t threads = M * (N / 4);
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks >= (1ll << 31)) return hipErrorInvalidValue;
#define MX_REDUCE(S)                                                                                         \
  case S:                                                                                                    \
    hipLaunchKernelGGL(splitk_reduce_kernel<S>, dim3((unsigned)blocks), dim3(256), 0, stream, ws, M, N, bias, \
                       bias_f32, c, c_f32, ldc);                                                             \
    break;
  switch (split_k) {
    MX_REDUCE(2)
    MX_REDUCE(3)
    MX_REDUCE(4)
    MX_REDUCE(5)
    MX_REDUCE(6)
    MX_REDUCE(7)
    MX_REDUCE(8)
    MX_REDUCE(9)
    MX_REDUCE(10)
    MX_REDUCE(11)
    MX_REDUCE(12)
    MX_REDUCE(13)
    MX_REDUCE(14)
    MX_REDUCE(15)
    MX_REDUCE(16)
    default: return hipErrorInvalidValue;
  }
#undef MX_REDUCE
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, int fmt, int mode, int epi, hipStream_t stream) {
  switch (fmt) {
    case kE2M1: return launch_fmt<kE2M1>(p, mode, epi, stream);
    case kE2M3: return launch_fmt<kE2M3>(p, mode, epi, stream);
    case kE4M3: return launch_fmt<kE4M3>(p, mode, epi, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mx
