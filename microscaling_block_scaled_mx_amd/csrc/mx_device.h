// Device-side building blocks of libmx (gfx950): bf16 conversion, E8M0 scale
// selection, E2M1/E2M3/E4M3 encoding, bit packing, the 32-point Hadamard
// butterfly and the activation prologues.  Compiled with -ffp-contract=off:
// every float operation below is one binary32 operation, rounded to nearest
// even, so the results are reproducible to the bit.
//
// Page references (by title):
//   [P1] "feat(mxfp6): MXFP6 (E2M3) Flux linears, a fused MLP, and the MLPerf
//        recipe" (Primus pull request 1064)
//   [P3] "MXFP4 training for Flux models" (ROCm Primus technical guide)
//   [P4] "MXFP8 cudnn-fe Swiglu fused Grouped MLP fwd/bwd and wgrad group
//        gemm" (ao pull request 5)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

enum Fmt { kE2M1 = 1, kE2M3 = 2, kE4M3 = 3 };
enum ScaleMode { kFloor = 0, kRceil = 1 };
enum Prologue { kIdentity = 0, kGelu = 1, kDGelu = 2, kSwiglu = 3, kDSwiglu = 4 };

template <int FMT> struct FmtTraits;
// E2M1: s|e2|m1, bias 1, largest 6.0 (code 7), sign bit 3.
template <> struct FmtTraits<kE2M1> {
  static constexpr int kBits = 4, kMant = 1, kEmin = 0, kEmaxElem = 2;
  static constexpr uint32_t kMaxCode = 7, kSign = 0x8;
};
// E2M3: s|e2|m3, bias 1, largest 7.5 (code 31), sign bit 5.
template <> struct FmtTraits<kE2M3> {
  static constexpr int kBits = 6, kMant = 3, kEmin = 0, kEmaxElem = 2;
  static constexpr uint32_t kMaxCode = 31, kSign = 0x20;
};
// E4M3 ("fn"): s|e4|m3, bias 7, largest 448 (code 0x7e), no infinities.
template <> struct FmtTraits<kE4M3> {
  static constexpr int kBits = 8, kMant = 3, kEmin = -6, kEmaxElem = 8;
  static constexpr uint32_t kMaxCode = 0x7e, kSign = 0x80;
};

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// binary32 -> bf16 bits, nearest-even; NaN stays NaN (quiet bit set).  The
// gfx950 conversion instruction follows exactly this rule (checked against
// (u + 0x7fff + lsb) >> 16, NaN -> (u >> 16) | 0x40, on all 2^32 inputs).
typedef __bf16 mx_bf16x2 __attribute__((ext_vector_type(2)));
typedef float mx_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const mx_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, mx_bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }
// Round through bf16 and back.
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(pack_bf16x2(f, 0.0f) << 16); }

// ------------------------------------------------------------------ E8M0
// Scale byte from the block's amax, given as the bit pattern of |amax| in
// binary32.  For non-negative floats integer order is value order and every
// NaN pattern sorts above +Inf, so a plain unsigned max over |x| bits is a
// NaN-propagating amax ([P4] commit messages).
//   NaN/Inf block     -> 0xff.
//   FLOOR: X = floor(log2 amax) - emax_elem  (exponent field; a subnormal
//          or zero amax falls under the low clamp anyway).
//   RCEIL: X = smallest integer with 448 * 2^X >= amax.  With amax = m*2^E,
//          m in [1,2): 448*2^(E-8) = 1.75*2^E, so X = E - 8 + (m > 1.75);
//          exact, no division ([P4]: the scale's E8M0 conversion rounds up).
//   X clamped to [-127, 127]; byte = X + 127.
template <int FMT, int MODE>
__device__ __forceinline__ uint32_t scale_byte(uint32_t amax_bits) {
  int ef = (int)(amax_bits >> 23);
  int X;
  if (MODE == kRceil) {
    X = ef - 127 - 8 + ((amax_bits & 0x7fffffu) > 0x600000u ? 1 : 0);
  } else {
    X = ef - 127 - FmtTraits<FMT>::kEmaxElem;
  }
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  return amax_bits >= 0x7f800000u ? 0xffu : (uint32_t)(X + 127);
}


// ------------------------------------------------------------------ Hadamard
// Normalised 32-point Walsh-Hadamard rotation in Sylvester order ([P1]
// description: mandatory for MXFP6, folded into the packer).  Radix-2
// butterfly, strides 1, 2, 4, 8, 16 (a+b, a-b), then one multiply by
// fl32(1/sqrt(32)) = 0x3e3504f3.
__device__ __forceinline__ void hadamard32(float (&y)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
    }
  }
  const float c = __uint_as_float(0x3e3504f3u);
#pragma unroll
  for (int i = 0; i < 32; ++i) y[i] = y[i] * c;
}

// ------------------------------------------------------------------ quantize one block
// v: 32 values (prologue applied, bf16-rounded, rotated if asked).
// Returns the scale byte; fills the packed words (E2M1 4 dwords, element 2j
// in the low nibble of byte j; E2M3 6 dwords, a little-endian 6-bit stream;
// E4M3 8 dwords, one byte per element).
//
// The codes come from the gfx950 scaled conversions, which compute x / 2^X
// exactly and round it to the format's nearest code, ties to the even code,
// saturating at the largest magnitude and keeping the sign (-0 included).
// That was checked against the nearest-even encoding rule over every code,
// every midpoint and its neighbours, saturation, signed zeros and
// denormals.  Two adjustments: E4M3 returns NaN past 448 instead of
// saturating, so a FLOOR-scaled block (where |x| / 2^X < 512) is clamped to
// +-448 * 2^X first; and 2^-127 is not a normal binary32, so a block with
// X = -127 is converted as (x * 2^64) / 2^-63.  A NaN/Inf block gets zero
// codes.
template <int FMT, int MODE>
__device__ __forceinline__ uint32_t quant_block(const float (&v)[32], uint32_t (&w)[FmtTraits<FMT>::kBits]) {
  [[maybe_unused]] constexpr int B = FmtTraits<FMT>::kBits;
  // amax of |v| on the bit patterns: positive values (and +NaN / +Inf)
  // order as signed integers, negative ones as unsigned integers above
  // every positive one, so the signed maximum (from 0) finds the largest
  // positive pattern and the unsigned maximum, sign cleared, the largest
  // negative one (or the same positive one if there is none)
  int32_t mpos = 0;
  uint32_t mneg = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t b = __float_as_uint(v[i]);
    mpos = mpos > (int32_t)b ? mpos : (int32_t)b;
    mneg = mneg > b ? mneg : b;
  }
  const uint32_t amax = (uint32_t)mpos > (mneg & 0x7fffffffu) ? (uint32_t)mpos : (mneg & 0x7fffffffu);
  const uint32_t s = scale_byte<FMT, MODE>(amax);
#if defined(__HIP_DEVICE_COMPILE__)
  const bool tiny = s == 0u;
  const float sc = __uint_as_float((tiny ? 64u : (s == 0xffu ? 127u : s)) << 23);  // 2^X (2^-63 if tiny)
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = v[i];
  if (__builtin_amdgcn_ballot_w64(tiny) != 0) {  // rare: only a wavefront holding a tiny block pays
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = tiny ? v[i] * 0x1p64f : v[i];
  }
  if constexpr (FMT == kE4M3 && MODE == kFloor) {
    const float bound = 448.0f * sc;
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __builtin_fminf(__builtin_fmaxf(x[i], -bound), bound);
  }
  if constexpr (FMT == kE2M1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t q = 0u;
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, x[8 * d + 0], x[8 * d + 1], sc, 0);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, x[8 * d + 2], x[8 * d + 3], sc, 1);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, x[8 * d + 4], x[8 * d + 5], sc, 2);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(q, x[8 * d + 6], x[8 * d + 7], sc, 3);
      w[d] = q;
    }
  } else if constexpr (FMT == kE4M3) {
    typedef short s2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      s2 q = {0, 0};
      q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q, x[4 * d + 0], x[4 * d + 1], sc, false);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q, x[4 * d + 2], x[4 * d + 3], sc, true);
      w[d] = __builtin_bit_cast(uint32_t, q);
    }
  } else {
    // the conversion interleaves its two 16-value operands (slot 2i <- a[i],
    // slot 2i + 1 <- b[i]): even elements go in a, odd ones in b
    typedef float f16v __attribute__((ext_vector_type(16)));
    typedef int i6v __attribute__((ext_vector_type(6)));
    f16v a, b;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      a[i] = x[2 * i];
      b[i] = x[2 * i + 1];
    }
    // The conversion's 6-dword result must not share registers with its
    // 32 source dwords or its scale: with the result placed two registers
    // below the sources (an allocation the compiler can choose), most codes
    // of the block came out wrong on gfx950.  The early-clobber output
    // keeps the result apart from every input.
    i6v q;
    asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(q) : "v"(a), "v"(b), "v"(sc));
#pragma unroll
    for (int d = 0; d < 6; ++d) w[d] = (uint32_t)q[d];
  }
  if (s == 0xffu) {
#pragma unroll
    for (int d = 0; d < B; ++d) w[d] = 0u;
  }
#endif
  return s;
}

// ------------------------------------------------------------------ LDS tiles
// A bf16 tile in LDS, row-major with `pitch` bytes per row (a multiple of 8).
// Row block: 32 consecutive bf16 of one row (8-byte aligned start).
__device__ __forceinline__ void lds_row_block(const uint8_t* tile, int pitch, int row, int col0, float (&v)[32]) {
  const uint2* src = reinterpret_cast<const uint2*>(tile + row * pitch + col0 * 2);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint2 q = src[j];
    v[4 * j + 0] = bf16_lo(q.x);
    v[4 * j + 1] = bf16_hi(q.x);
    v[4 * j + 2] = bf16_lo(q.y);
    v[4 * j + 3] = bf16_hi(q.y);
  }
}
// Column block: rows row0..row0+31 of one column.
__device__ __forceinline__ void lds_col_block(const uint8_t* tile, int pitch, int row0, int col, float (&v)[32]) {
  const uint16_t* src = reinterpret_cast<const uint16_t*>(tile + row0 * pitch) + col;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(src[i * (pitch / 2)]);
}

// Store one block's packed codes into its K group (group base g, block
// blk = 0..3 of the group, row = the packed operand's row): E2M1 16 B at
// 16 blk, E4M3 32 B at 32 blk, E2M3 its first 16 B at 16 blk and its last
// 8 B at 64 + 8 (blk ^ ((row >> 4) & 1)) -- rows with bit 4 set swap the two
// 8-byte tails that share a 16-byte chunk, so that the 8-byte reads of 32
// consecutive rows fall in distinct LDS banks.
template <int FMT>
__device__ __forceinline__ void store_block(uint8_t* g, int blk, int64_t row,
                                            const uint32_t (&w)[FmtTraits<FMT>::kBits]) {
  if constexpr (FMT == kE2M1) {
    *reinterpret_cast<uint4*>(g + 16 * blk) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (FMT == kE2M3) {
    *reinterpret_cast<uint4*>(g + 16 * blk) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint2*>(g + 64 + 8 * (blk ^ (int)((row >> 4) & 1))) = make_uint2(w[4], w[5]);
  } else {
    uint4* d = reinterpret_cast<uint4*>(g + 32 * blk);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// Zero codes of one block (a pad block of a partial K group).
template <int FMT>
__device__ __forceinline__ void zero_block(uint8_t* g, int blk, int64_t row) {
  uint32_t w[FmtTraits<FMT>::kBits];
#pragma unroll
  for (int i = 0; i < FmtTraits<FMT>::kBits; ++i) w[i] = 0u;
  store_block<FMT>(g, blk, row, w);
}

// Quantize 32 values and write codes (block blk of group g of the packed
// operand's row `row`) + scale byte.
template <int FMT, int MODE, int HAD>
__device__ __forceinline__ void quant_store(float (&v)[32], uint8_t* g, int blk, int64_t row, uint8_t* scale) {
  if constexpr (HAD) hadamard32(v);
  uint32_t w[FmtTraits<FMT>::kBits];
  const uint32_t s = quant_block<FMT, MODE>(v, w);
  store_block<FMT>(g, blk, row, w);
  *scale = (uint8_t)s;
}

// ------------------------------------------------------------------ stochastic rounding (E2M1)
// MXFP4 gradient packs may round stochastically ([P3] Overview, configuration
// table: SR of the FP4 gradient quantization).  The random word of element
// i of a packed operand is word i % 4 of Philox4x32-10 (Salmon, Moraes,
// Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011)
// at counter (i/4 low, i/4 high, axis, 0), key (seed low, seed high); axis
// 0 = rowwise operand, 1 = columnwise.  One round multiplies counter words 0
// and 2 by 0xD2511F53 and 0xCD9E8D57 (full 64-bit products) and recombines
// them with words 1, 3 and the key; the key advances by 0x9E3779B9 and
// 0xBB67AE85 between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32 x 32 -> 64-bit product each (both halves from one instruction)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = (uint32_t)p1;
    c[2] = n2;
    c[3] = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// E2M1 code of v = x / 2^X (exact) rounded stochastically with the random
// word r: |v| >= 6 saturates; otherwise, with grid neighbours lo <= |v| < hi
// (spacing 0.5 below 2, 1 below 4, else 2) and t = (|v| - lo) / (hi - lo),
// the magnitude is hi iff (r >> 8) < floor(t * 2^24).  Every step is exact
// in binary32.  The sign is kept (-0 included).
__device__ __forceinline__ uint32_t e2m1_sr_code(float v, uint32_t r) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
  const float a = __builtin_fabsf(v);
  // the three spacing regimes as selects, not branches (|v| < 8 here)
  const bool r1 = a < 2.0f, r2 = a < 4.0f;
  const float f2 = __builtin_floorf(a * 2.0f), f1 = __builtin_floorf(a);
  const uint32_t clo = r1 ? (uint32_t)f2 : (r2 ? 2u + (uint32_t)f1 : 6u);
  const float lo = r1 ? f2 * 0.5f : (r2 ? f1 : 4.0f);
  const float inv = r1 ? 2.0f : (r2 ? 1.0f : 0.5f);
  const uint32_t k = (uint32_t)(((a - lo) * inv) * 16777216.0f);
  const uint32_t c = a >= 6.0f ? 7u : clo + ((r >> 8) < k ? 1u : 0u);
  return sign | c;
}

// One E2M1 block with stochastic rounding: the FLOOR scale of nearest
// packing, codes by e2m1_sr_code with the words of elements i0 .. i0 + 31
// (i0 a multiple of 32).  A NaN/Inf block gets zero codes.
__device__ __forceinline__ void quant_store_sr(const float (&v)[32], uint8_t* g, int blk, int64_t row,
                                               uint8_t* scale, uint64_t seed, uint32_t axis, uint64_t i0) {
  uint32_t amax = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t b = __float_as_uint(v[i]) & 0x7fffffffu;
    amax = amax > b ? amax : b;
  }
  const uint32_t s = scale_byte<kE2M1, kFloor>(amax);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (s != 0xffu) {
    const int nx = 127 - (int)s;  // -X
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t q = (i0 >> 2) + (uint64_t)j;
      uint32_t c[4] = {(uint32_t)q, (uint32_t)(q >> 32), axis, 0u};
      philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int el = 4 * j + e;
        w[el / 8] |= e2m1_sr_code(__builtin_ldexpf(v[el], nx), c[e]) << (4 * (el % 8));
      }
    }
  }
  store_block<kE2M1>(g, blk, row, w);
  *scale = (uint8_t)s;
}

// ------------------------------------------------------------------ prologue math
// Own exp (binary32), the library's contract: Cody-Waite reduction
// n = rint(x * LOG2E), r = fma(-n, LN2_HI, x) (exact product: LN2_HI is ln 2
// cut to 16 significant bits), r = fma(-n, LN2_LO, r), then the degree-7
// Taylor polynomial (1/k! rounded to binary32) in Horner order, one fused
// multiply-add per step, scaled by 2^n.  x < -87 -> +0 (results stay
// normal), x > 89 -> +inf, NaN -> NaN.  mx_exp_core is the arithmetic
// without the range checks.
__device__ __forceinline__ float mx_exp_core(float x) {
  const float LOG2E = 0x1.715476p+0f;   // fl32(1/ln 2)
  const float LN2_HI = 0x1.62e4p-1f;     // 0.693145751953125
  const float LN2_LO = 0x1.7f7d1cp-20f;  // fl32(ln 2 - LN2_HI)
  const float P2 = 0x1.0p-1f, P3 = 0x1.555556p-3f, P4 = 0x1.555556p-5f;
  const float P5 = 0x1.111112p-7f, P6 = 0x1.6c16c2p-10f, P7 = 0x1.a01a02p-13f;
  const float n = __builtin_rintf(x * LOG2E);
  float r = __builtin_fmaf(-n, LN2_HI, x);
  r = __builtin_fmaf(-n, LN2_LO, r);
  float p = P7;
  p = __builtin_fmaf(r, p, P6);
  p = __builtin_fmaf(r, p, P5);
  p = __builtin_fmaf(r, p, P4);
  p = __builtin_fmaf(r, p, P3);
  p = __builtin_fmaf(r, p, P2);
  p = __builtin_fmaf(r, p, 1.0f);
  p = __builtin_fmaf(r, p, 1.0f);
  return __builtin_ldexpf(p, (int)n);
}
__device__ __forceinline__ float mx_exp(float x) {
  float res = mx_exp_core(x);
  res = (x > 89.0f) ? __builtin_inff() : res;
  res = (x < -87.0f) ? 0.0f : res;
  return (x != x) ? x : res;
}
// mx_exp for x >= 0 or NaN (x < -87 cannot occur, so its check is left out).
__device__ __forceinline__ float mx_exp_nonneg(float x) {
  float res = mx_exp_core(x);
  res = (x > 89.0f) ? __builtin_inff() : res;
  return (x != x) ? x : res;
}

// tanh-GELU pieces.  u = K0*fma(K1, (x*x)*x, x); q = 2/(exp(2|u|)+1);
// 1 + tanh(u) = q (u < 0) or 2 - q (u >= 0); 1 - tanh(u)^2 = q*(2-q).
// K0 = fl32(sqrt(2/pi)), K1 = fl32(0.044715).
__device__ __forceinline__ float gelu_u(float x) {
  const float K0 = 0x1.988454p-1f, K1 = 0x1.6e4e26p-5f;
  float x3 = (x * x) * x;
  float inner = __builtin_fmaf(K1, x3, x);
  return K0 * inner;
}
// n / d for n = 1 or 2 and d >= 1, rounded to nearest even: the hardware
// reciprocal and one FMA refinement, which equals the IEEE division bit for
// bit for every binary32 d in [1, 2^126) (checked exhaustively on gfx950,
// for both numerators).  Past that the quotient is subnormal and the
// reciprocal flushes it, so a wavefront holding such a d (or a NaN, or
// +inf) takes the IEEE division for those lanes.
__device__ __forceinline__ float div_small(float n, float d) {
#if defined(__HIP_DEVICE_COMPILE__)
  const float r = __builtin_amdgcn_rcpf(d);
  const float q0 = n * r;
  const float e = __builtin_fmaf(-d, q0, n);
  float q = __builtin_fmaf(e, r, q0);
  const bool slow = !(d < 0x1p126f);
  if (__builtin_amdgcn_ballot_w64(slow) != 0) q = slow ? n / d : q;
  return q;
#else
  return n / d;
#endif
}

__device__ __forceinline__ float gelu_q(float u) {
  float e = mx_exp_nonneg(2.0f * __builtin_fabsf(u));
  return div_small(2.0f, e + 1.0f);
}

// a = bf16((0.5*x) * (1 + tanh u))
__device__ __forceinline__ float gelu_bf16(float x) {
  float u = gelu_u(x);
  float q = gelu_q(u);
  float opt = (u < 0.0f) ? q : (2.0f - q);
  return round_bf16((0.5f * x) * opt);
}

// dh = bf16(da * (0.5*(1+tanh u) + (0.5*x) * ((q*(2-q)) * (K0*fma(3*K1, x*x, 1)))))
// with the second term taken as 0 when q*(2-q) == 0.
__device__ __forceinline__ float dgelu_bf16(float da, float x) {
  const float K0 = 0x1.988454p-1f, K1x3 = 0x1.12ba9cp-3f;  // fl32(3 * fl32(0.044715))
  float u = gelu_u(x);
  float q = gelu_q(u);
  float opt = (u < 0.0f) ? q : (2.0f - q);
  float w = q * (2.0f - q);
  float first = 0.5f * opt;
  float second = (0.5f * x) * (w * (K0 * __builtin_fmaf(K1x3, x * x, 1.0f)));
  second = (w == 0.0f) ? 0.0f : second;
  return round_bf16(da * (first + second));
}

// SwiGLU on [gate | up] ([P4] commit messages: sigmoid as 1/(1+exp(-x))).
__device__ __forceinline__ float sigmoid_mx(float g) { return div_small(1.0f, 1.0f + mx_exp(-g)); }
// The same value with the plain IEEE division: the dSwiGLU epilogue of the
// grouped GEMM interleaves its loads of H with this arithmetic, and there
// the reciprocal path's wavefront-uniform branch measured slower.
__device__ __forceinline__ float sigmoid_ieee(float g) { return 1.0f / (1.0f + mx_exp(-g)); }
__device__ __forceinline__ float swiglu_bf16(float g, float u) {
  float s = sigmoid_mx(g);
  return round_bf16((g * s) * u);
}
// d_gate = bf16((dz*u) * (s*(1 + g*(1-s)))),  d_up = bf16(dz*(g*s)).
__device__ __forceinline__ float dswiglu_gate_bf16(float dz, float g, float u) {
  float s = sigmoid_ieee(g);
  return round_bf16((dz * u) * (s * (1.0f + g * (1.0f - s))));
}
__device__ __forceinline__ float dswiglu_up_bf16(float dz, float g) {
  float s = sigmoid_ieee(g);
  return round_bf16(dz * (g * s));
}
// Both of one element, the sigmoid formed once (bitwise the two above: the
// reciprocal division equals the IEEE quotient for every divisor it sees).
__device__ __forceinline__ void dswiglu_pair_bf16(float dz, float g, float u, float& d_gate, float& d_up) {
  const float s = sigmoid_mx(g);
  d_up = round_bf16(dz * (g * s));
  d_gate = round_bf16((dz * u) * (s * (1.0f + g * (1.0f - s))));
}

}  // namespace mx
