/*
 * mx_oracle.c -- plain, slow, scalar CPU oracle for OCP-microscaling (MX)
 * quantize-and-GEMM.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg are the only callers.  Nothing in the
 * GPU library links, includes or calls this file, and this file shares no
 * code, header, table or constant with the GPU library.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 *        (no FMA contraction: every float operation below is one IEEE-754
 *        binary32 or binary64 operation, rounded to nearest-even).
 *
 * Sources.  The pages this follows are
 *   [P1] "feat(mxfp6): MXFP6 (E2M3) Flux linears, a fused MLP, and the MLPerf
 *        recipe" (Primus pull request 1064): description, commit messages,
 *        Summary, Test plan.
 *   [P3] "MXFP4 training for Flux models" (ROCm Primus technical guide):
 *        Overview, Troubleshooting.
 *   [P4] "MXFP8 cudnn-fe Swiglu fused Grouped MLP fwd/bwd and wgrad group
 *        gemm" (ao pull request 5): commit messages.
 * The pages name the element formats but do not spell out their bit
 * encodings; those follow the OCP Microscaling Formats (MX) v1.0
 * specification, which defines E2M1, E2M3, E4M3 and E8M0.
 *
 * Where the pages leave a step open, the reading taken is stated at that
 * step.  Every function here is pinned by tests against values fixed by the
 * pages or by mathematics (see the test files); the prologue functions
 * (own exp, tanh, GELU, SwiGLU) are a contract shared with the GPU path and
 * are pinned only against libm / high-precision references within stated
 * error bounds.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E2M1 1
#define ORC_E2M3 2
#define ORC_E4M3 3

#define ORC_FLOOR 0
#define ORC_RCEIL 1

#define ORC_PRO_IDENTITY 0
#define ORC_PRO_GELU 1
#define ORC_PRO_DGELU 2
#define ORC_PRO_SWIGLU 3
#define ORC_PRO_DSWIGLU 4

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32                                                        */
/* ------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float orc_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* Round an fp32 value to bf16, nearest-even; NaN stays NaN (made quiet). */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u = f32_to_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* Element formats (OCP MX v1.0 encodings; the pages name E2M1 for     */
/* MXFP4 [P3 Overview], E2M3 for MXFP6 [P1 Summary], E4M3 for MXFP8    */
/* [P4 commit messages]).                                              */
/* ------------------------------------------------------------------ */

int orc_code_bits(int fmt) { return fmt == ORC_E2M1 ? 4 : fmt == ORC_E2M3 ? 6 : 8; }

/* Largest positive finite code of each format. */
static unsigned max_code(int fmt) {
  return fmt == ORC_E2M1 ? 0x7u : fmt == ORC_E2M3 ? 0x1fu : 0x7eu;
}
static unsigned sign_bit(int fmt) {
  return fmt == ORC_E2M1 ? 0x8u : fmt == ORC_E2M3 ? 0x20u : 0x80u;
}

/* Decode one element code to its exact value (as a double).
 * E2M1: s | e(2) | m(1), bias 1.  E2M3: s | e(2) | m(3), bias 1.
 * E4M3 ("fn"): s | e(4) | m(3), bias 7, no infinities, 0x7f/0xff NaN.
 * Exponent field 0 encodes subnormals m * 2^(1-bias) / 2^mbits. */
double orc_decode(int fmt, unsigned code) {
  int ebits, mbits, bias;
  if (fmt == ORC_E2M1) { ebits = 2; mbits = 1; bias = 1; }
  else if (fmt == ORC_E2M3) { ebits = 2; mbits = 3; bias = 1; }
  else { ebits = 4; mbits = 3; bias = 7; }
  unsigned nbits = 1 + ebits + mbits;
  code &= (1u << nbits) - 1u;
  int s = (code >> (nbits - 1)) & 1u;
  unsigned e = (code >> mbits) & ((1u << ebits) - 1u);
  unsigned m = code & ((1u << mbits) - 1u);
  if (fmt == ORC_E4M3 && e == 15 && m == 7) return NAN;
  double v;
  if (e == 0) v = ldexp((double)m, 1 - bias - mbits);
  else v = ldexp((double)((1u << mbits) | m), (int)e - bias - mbits);
  return s ? -v : v;
}

/* Encode a finite value: round to the nearest representable magnitude,
 * ties to the code whose mantissa LSB is 0 (nearest-even), saturating at the
 * largest finite magnitude; the sign is kept, so a negative value that rounds
 * to zero gives the negative-zero code.  Codes 0..max_code are ordered by
 * magnitude, so the search below is a plain bisection over the code order. */
unsigned orc_encode(int fmt, double v) {
  unsigned sgn = (signbit(v) != 0) ? sign_bit(fmt) : 0u;
  double a = fabs(v);
  unsigned top = max_code(fmt);
  if (a >= orc_decode(fmt, top)) return sgn | top;
  /* largest code lo with decode(lo) <= a */
  unsigned lo = 0, hi = top;
  while (hi - lo > 1) {
    unsigned mid = (lo + hi) / 2;
    if (orc_decode(fmt, mid) <= a) lo = mid; else hi = mid;
  }
  double dlo = a - orc_decode(fmt, lo), dhi = orc_decode(fmt, hi) - a;
  unsigned c;
  if (dlo < dhi) c = lo;
  else if (dhi < dlo) c = hi;
  else c = (lo & 1u) ? hi : lo;
  return sgn | c;
}

/* ------------------------------------------------------------------ */
/* E8M0 shared exponent: one per block of 32 [P3 Overview; P1 Summary]. */
/* byte b encodes 2^(b-127); 0xff is NaN.                              */
/* ------------------------------------------------------------------ */

/* Exponent of the largest power of two <= x, for finite x > 0, read from
 * the binary representation (exact, subnormals included). */
static int floor_log2_f32(float x) {
  int e;
  double f = frexp((double)x, &e); /* x = f * 2^e, f in [0.5, 1) */
  (void)f;
  return e - 1;
}

/* FLOOR selection for MXFP4 and MXFP6: the pages only say E8M0 block-of-32
 * scales; the reading taken is the OCP MX v1.0 default conversion, which
 * takes X = floor(log2(amax)) - emax_elem with emax_elem the exponent of the
 * element format's largest normal (2 for E2M1: 6 = 1.5*2^2; 2 for E2M3:
 * 7.5 = 1.875*2^2; 8 for E4M3: 448 = 1.75*2^8).  Clamped to [-127, 127].
 * amax == 0 has no finite log; the clamp's low end (byte 0x00) is taken.
 * A NaN or infinite amax gives the NaN scale 0xff. */
unsigned orc_scale_floor(int fmt, float amax) {
  if (isnan(amax) || isinf(amax)) return 0xffu;
  int emax_elem = (fmt == ORC_E4M3) ? 8 : 2;
  int e;
  if (amax == 0.0f) e = -127;
  else e = floor_log2_f32(amax) - emax_elem;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return (unsigned)(e + 127);
}

/* RCEIL selection for MXFP8 [P4 commit messages: the E8M0 conversion of the
 * scale rounds upward]: q = fl32(amax / 448) in binary32, then the smallest
 * power of two >= q.  Clamped to [-127, 127]; q == 0 gives 0x00; NaN or
 * infinite amax gives 0xff. */
unsigned orc_scale_rceil(float amax) {
  if (isnan(amax) || isinf(amax)) return 0xffu;
  volatile float q = amax / 448.0f; /* one binary32 division */
  if (q == 0.0f) return 0x00u;
  int e = floor_log2_f32(q);
  if (ldexp(1.0, e) != (double)q) e += 1; /* not a power of two: round up */
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return (unsigned)(e + 127);
}

/* ------------------------------------------------------------------ */
/* Own exp / tanh and the activation prologues.                         */
/* [P1 description/Summary]: the fused MLP reproduces the unfused path     */
/* exactly; the unfused path materialises bf16 tensors.  [P4 commit       */
/* messages]: sigmoid is formed as 1/(1+exp(-x)).  The pages fix no exp   */
/* implementation; to make both sides bit-identical, exp is our own:      */
/* Cody-Waite range reduction with a two-part ln2 and a degree-7 Taylor  */
/* polynomial (coefficients 1/k!, rounded to binary32), Horner order.     */
/* Every step is one binary32 operation: a product, a sum, or a fused     */
/* multiply-add (one rounding of a*b + c, C99 fmaf), as named below.      */
/* ------------------------------------------------------------------ */

/* Constants of the exp contract, each derived here from its definition:
 *   LOG2E  = fl32(1/ln 2)
 *   LN2_HI = ln 2 truncated to 16 significant bits (so n*LN2_HI is exact
 *            for |n| <= 256)
 *   LN2_LO = fl32(ln 2 - LN2_HI) */
static float c_log2e(void) { return (float)(1.0 / 0.69314718055994530941723212145818); }
static float c_ln2_hi(void) {
  double ln2 = 0.69314718055994530941723212145818;
  return (float)(floor(ldexp(ln2, 16)) / 65536.0);
}
static float c_ln2_lo(void) {
  double ln2 = 0.69314718055994530941723212145818;
  return (float)(ln2 - (double)c_ln2_hi());
}

/* exp(x) in binary32:
 *   x NaN -> NaN; x > 89 -> +inf; x < -87 -> +0 (the results in between
 *   stay normal; the activations only ever need exp of large negative
 *   arguments inside 1/(1+exp(.)), where 0 and a subnormal give the same).
 *   n = rint(x * LOG2E);
 *   r = fma(-n, LN2_HI, x)  (n*LN2_HI is exact, so this is x - n*LN2_HI);
 *   r = fma(-n, LN2_LO, r);
 *   p = 1/5040; then p = fma(r, p, c) for c = 1/720, 1/120, 1/24, 1/6, 1/2,
 *   1, 1 in turn (Horner order, one rounding per step);
 *   result = p * 2^n (exact power-of-two scaling), +inf when it overflows. */
float orc_exp(float x) {
  if (isnan(x)) return x;
  if (x < -87.0f) return 0.0f;
  if (x > 89.0f) return INFINITY;
  const float L2E = c_log2e(), LH = c_ln2_hi(), LL = c_ln2_lo();
  const float k2 = (float)(1.0 / 2.0), k3 = (float)(1.0 / 6.0), k4 = (float)(1.0 / 24.0);
  const float k5 = (float)(1.0 / 120.0), k6 = (float)(1.0 / 720.0), k7 = (float)(1.0 / 5040.0);
  float t = x * L2E;
  float n = rintf(t);
  float r = fmaf(-n, LH, x);
  r = fmaf(-n, LL, r);
  float p = k7;
  p = fmaf(r, p, k6);
  p = fmaf(r, p, k5);
  p = fmaf(r, p, k4);
  p = fmaf(r, p, k3);
  p = fmaf(r, p, k2);
  p = fmaf(r, p, 1.0f);
  p = fmaf(r, p, 1.0f);
  double res = ldexp((double)p, (int)n); /* exact: p has 24 bits */
  if (res > 3.4028234663852886e38) return INFINITY;
  return (float)res;
}

/* The tanh that the GELU needs only enters as 1 + tanh(u) and 1 - tanh(u)^2.
 * With q = 2/(exp(2|u|) + 1) (so tanh|u| = 1 - q):
 *   1 + tanh(u) = q        for u < 0,   2 - q   for u >= 0,
 *   1 - tanh(u)^2 = q * (2 - q)         for all u.
 * Written this way neither tail cancels.  exp overflowing to +inf gives
 * q = 0 (tanh = +-1); NaN propagates. */
static float gelu_q(float u) {
  float e = orc_exp(2.0f * fabsf(u));
  return 2.0f / (e + 1.0f);
}

float orc_one_plus_tanh(float u) {
  float q = gelu_q(u);
  return (u < 0.0f) ? q : (2.0f - q);
}

/* tanh-approximation GELU constants: K0 = fl32(sqrt(2/pi)), K1 = fl32(0.044715). */
static float c_k0(void) { return (float)sqrt(2.0 / 3.14159265358979323846264338327950288); }
static float c_k1(void) { return (float)0.044715; }

/* u = K0 * fma(K1, (x*x)*x, x) */
static float gelu_u(float x) {
  const float K0 = c_k0(), K1 = c_k1();
  float x3 = (x * x) * x;
  float inner = fmaf(K1, x3, x);
  return K0 * inner;
}

/* a = bf16((0.5*x) * (1 + tanh(u))) */
uint16_t orc_gelu_bf16(uint16_t hb) {
  float x = orc_bf16_to_f32(hb);
  float a = (0.5f * x) * orc_one_plus_tanh(gelu_u(x));
  return orc_f32_to_bf16(a);
}

/* Derivative of the tanh-GELU above, times the incoming gradient:
 *   dg = 0.5*(1+tanh u) + (0.5*x) * ((q*(2-q)) * (K0 * fma(3*K1, x*x, 1)))
 *   dh = bf16(da * dg)
 * When q*(2-q) is exactly 0 the second term is taken as 0 (it avoids 0*inf
 * for huge |x|). */
uint16_t orc_dgelu_bf16(uint16_t dab, uint16_t hb) {
  float x = orc_bf16_to_f32(hb), da = orc_bf16_to_f32(dab);
  const float K0 = c_k0(), K1 = c_k1();
  const float K1x3 = 3.0f * K1;
  float u = gelu_u(x);
  float q = gelu_q(u);
  float opt = (u < 0.0f) ? q : (2.0f - q);
  float w = q * (2.0f - q);
  float first = 0.5f * opt;
  float second;
  if (w == 0.0f) second = 0.0f;
  else second = (0.5f * x) * (w * (K0 * fmaf(K1x3, x * x, 1.0f)));
  float dg = first + second;
  return orc_f32_to_bf16(da * dg);
}

/* SwiGLU on a [gate | up] pair: s = 1/(1+exp(-g)); z = bf16((g*s)*u). */
uint16_t orc_swiglu_bf16(uint16_t gb, uint16_t ub) {
  float g = orc_bf16_to_f32(gb), u = orc_bf16_to_f32(ub);
  float s = 1.0f / (1.0f + orc_exp(-g));
  return orc_f32_to_bf16((g * s) * u);
}

/* dSwiGLU: d_up = bf16(dz*(g*s)); d_gate = bf16((dz*u)*(s*(1 + g*(1-s)))). */
void orc_dswiglu_bf16(uint16_t dzb, uint16_t gb, uint16_t ub, uint16_t* dgate, uint16_t* dup) {
  float dz = orc_bf16_to_f32(dzb), g = orc_bf16_to_f32(gb), u = orc_bf16_to_f32(ub);
  float s = 1.0f / (1.0f + orc_exp(-g));
  *dup = orc_f32_to_bf16(dz * (g * s));
  *dgate = orc_f32_to_bf16((dz * u) * (s * (1.0f + g * (1.0f - s))));
}

/* ------------------------------------------------------------------ */
/* Hadamard-32 rotation (MXFP6 only) [P1 description, Summary: the       */
/* rotation is mandatory and folded into the packer].  The pages give     */
/* neither size, order nor normalisation; the reading taken: the 32-point */
/* Sylvester-ordered matrix H[i][j] = (-1)^popcount(i & j), one block of  */
/* 32 along the consuming GEMM's K, normalised by 1/sqrt(32) so that      */
/* H/sqrt(32) is orthogonal and both operands' rotations cancel in A.B^T. */
/* Arithmetic order (fixed so that results are reproducible to the bit):  */
/* S_i = sum_j H[i][j] x_j as a balanced pairwise tree over j in index    */
/* order, every add/sub rounded to binary32; r_i = fl32(S_i * c) with     */
/* c = fl32(1/sqrt(32)).                                                  */
/* ------------------------------------------------------------------ */

static float had_tree(const float* x, int i, int lo, int n) {
  if (n == 1) return x[lo];
  int half = n / 2;
  float a = had_tree(x, i, lo, half);
  float b = had_tree(x, i, lo + half, half);
  /* j in the upper half carries bit log2(half) of j; its sign is
   * (-1)^(that bit of i). */
  return (i & half) ? (a - b) : (a + b);
}

float orc_hadamard_c(void) { return (float)(1.0 / sqrt(32.0)); }

void orc_hadamard32(const float* x, float* r) {
  const float c = orc_hadamard_c();
  for (int i = 0; i < 32; ++i) r[i] = had_tree(x, i, 0, 32) * c;
}

/* ------------------------------------------------------------------ */
/* Packed layout in memory (the pages fix only a two-codes-per-byte fp4  */
/* type [P3 Troubleshooting] and the NT GEMM layout; the rest is this    */
/* library's reading): each operand row holds K codes, K-contiguous.     */
/*   E2M1: element 2j in the low nibble of byte j, 2j+1 in the high one. */
/*   E2M3: little-endian 6-bit stream; element j at bits [6j, 6j+6).     */
/*   E4M3: one byte per element.                                          */
/* Scales: one byte per 32-block, [rows][K/32].                          */
/* ------------------------------------------------------------------ */

int64_t orc_row_bytes(int fmt, int64_t k) { return k * orc_code_bits(fmt) / 8; }

void orc_put_code(uint8_t* row, int fmt, int64_t j, unsigned code) {
  int bits = orc_code_bits(fmt);
  if (bits == 8) { row[j] = (uint8_t)code; return; }
  int64_t bit = j * bits;
  for (int b = 0; b < bits; ++b) {
    int64_t pos = bit + b;
    uint8_t mask = (uint8_t)(1u << (pos & 7));
    if ((code >> b) & 1u) row[pos >> 3] |= mask;
    else row[pos >> 3] &= (uint8_t)~mask;
  }
}

unsigned orc_get_code(const uint8_t* row, int fmt, int64_t j) {
  int bits = orc_code_bits(fmt);
  if (bits == 8) return row[j];
  int64_t bit = j * bits;
  unsigned c = 0;
  for (int b = 0; b < bits; ++b) {
    int64_t pos = bit + b;
    c |= (unsigned)((row[pos >> 3] >> (pos & 7)) & 1u) << b;
  }
  return c;
}

/* ------------------------------------------------------------------ */
/* Quantize one block of 32 values (already prologue-applied and          */
/* bf16-rounded; rotated if requested): amax -> E8M0 -> cast.            */
/* amax propagates NaN [P4 commit messages].  A block whose amax is NaN   */
/* or infinite gets the NaN scale 0xff; the reading taken for its codes   */
/* (the pages are silent) is all +0.                                     */
/* ------------------------------------------------------------------ */

static void quant_block(const float* v, int fmt, int mode, unsigned* codes, unsigned* scale) {
  float amax = 0.0f;
  int has_nan = 0;
  for (int i = 0; i < 32; ++i) {
    if (isnan(v[i])) has_nan = 1;
    float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  if (has_nan) amax = NAN;
  unsigned s = (mode == ORC_RCEIL) ? orc_scale_rceil(amax) : orc_scale_floor(fmt, amax);
  *scale = s;
  if (s == 0xffu) {
    for (int i = 0; i < 32; ++i) codes[i] = 0u;
    return;
  }
  int e = (int)s - 127;
  for (int i = 0; i < 32; ++i) codes[i] = orc_encode(fmt, ldexp((double)v[i], -e));
}

/* Prologue output (bf16 bits) at logical element (r, c) of the quantized
 * tensor [R][C]:
 *   IDENTITY: x[r][c]                             x: [R][C]
 *   GELU:     gelu(x[r][c])                        x = h: [R][C]
 *   DGELU:    dgelu(da = x[r][c], h = aux[r][c])  x = da, aux = h: [R][C]
 *   SWIGLU:   swiglu(g = x[r][c], u = x[r][C+c])   x = H [gate|up]: [R][2C]
 *   DSWIGLU:  C = 2F, x = dz [R][F], aux = H [R][2F]:
 *             c <  F: d_gate(dz[r][c],   H[r][c],   H[r][F+c])
 *             c >= F: d_up  (dz[r][c-F], H[r][c-F], H[r][c]) */
static uint16_t prologue_at(const uint16_t* x, const uint16_t* aux, int64_t R, int64_t C, int pro,
                            int64_t r, int64_t c) {
  (void)R;
  switch (pro) {
    case ORC_PRO_GELU: return orc_gelu_bf16(x[r * C + c]);
    case ORC_PRO_DGELU: return orc_dgelu_bf16(x[r * C + c], aux[r * C + c]);
    case ORC_PRO_SWIGLU: return orc_swiglu_bf16(x[r * 2 * C + c], x[r * 2 * C + C + c]);
    case ORC_PRO_DSWIGLU: {
      int64_t F = C / 2;
      uint16_t dg, du;
      if (c < F) {
        orc_dswiglu_bf16(x[r * F + c], aux[r * C + c], aux[r * C + F + c], &dg, &du);
        return dg;
      }
      orc_dswiglu_bf16(x[r * F + (c - F)], aux[r * C + (c - F)], aux[r * C + c], &dg, &du);
      return du;
    }
    default: return x[r * C + c];
  }
}

/* Materialise the prologue output v [R][C] as bf16 bits. */
void orc_prologue(const uint16_t* x, const uint16_t* aux, int64_t R, int64_t C, int pro, uint16_t* v) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r)
    for (int64_t c = 0; c < C; ++c) v[r * C + c] = prologue_at(x, aux, R, C, pro, r, c);
}

/* Quantize a bf16 tensor [R][C] (after the prologue) into MX operands.
 *   row mode: blocks of 32 consecutive elements along dim 1 (1x32),
 *             output [R][C] codes + [R][C/32] scales.
 *   col mode: blocks of 32 consecutive rows of one column (32x1), written
 *             transposed, i.e. as a K-major operand [C][R] + [C][R/32].
 *   hadamard: rotate each block before amax (E2M3 only).
 *   colsum:   partials[b][c] = fp32 sum of the block's 32 prologue outputs
 *             (before rotation), rows 32b..32b+31 in increasing order from
 *             +0; sums[c] = fp32 sum of partials[0..R/32-1][c] in order.
 *             [P1 commit messages: the bias gradient is finished from the
 *             packer's per-column partials.]  The partial granularity (one
 *             32-row block) and order are this library's reading.
 * Any output pointer may be NULL.  R and C must be multiples of 32.
 * Returns 0 on success, nonzero on bad arguments. */
int orc_quantize(const uint16_t* x, const uint16_t* aux, int64_t R, int64_t C, int fmt, int mode,
                 int hadamard, int pro, uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                 uint8_t* col_scales, float* colsum_partials, float* colsum) {
  if (R % 32 || C % 32 || R < 0 || C < 0) return 1;
  if (fmt < ORC_E2M1 || fmt > ORC_E4M3) return 2;
  uint16_t* v = (uint16_t*)malloc((size_t)(R * C > 0 ? R * C : 1) * sizeof(uint16_t));
  if (!v) return 3;
  orc_prologue(x, aux, R, C, pro, v);
  int64_t rb = orc_row_bytes(fmt, C), cb = orc_row_bytes(fmt, R);
  if (row_codes) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
      for (int64_t b = 0; b < C / 32; ++b) {
        float blk[32], rot[32];
        unsigned codes[32], s;
        for (int i = 0; i < 32; ++i) blk[i] = orc_bf16_to_f32(v[r * C + b * 32 + i]);
        if (hadamard) { orc_hadamard32(blk, rot); memcpy(blk, rot, sizeof blk); }
        quant_block(blk, fmt, mode, codes, &s);
        row_scales[r * (C / 32) + b] = (uint8_t)s;
        for (int i = 0; i < 32; ++i) orc_put_code(row_codes + r * rb, fmt, b * 32 + i, codes[i]);
      }
    }
  }
  if (col_codes || colsum_partials || colsum) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
      float total = 0.0f;
      for (int64_t b = 0; b < R / 32; ++b) {
        float blk[32], rot[32];
        unsigned codes[32], s;
        float part = 0.0f;
        for (int i = 0; i < 32; ++i) {
          blk[i] = orc_bf16_to_f32(v[(b * 32 + i) * C + c]);
          part = part + blk[i];
        }
        if (colsum_partials) colsum_partials[b * C + c] = part;
        total = total + part;
        if (col_codes) {
          if (hadamard) { orc_hadamard32(blk, rot); memcpy(blk, rot, sizeof blk); }
          quant_block(blk, fmt, mode, codes, &s);
          col_scales[c * (R / 32) + b] = (uint8_t)s;
          for (int i = 0; i < 32; ++i) orc_put_code(col_codes + c * cb, fmt, b * 32 + i, codes[i]);
        }
      }
      if (colsum) colsum[c] = total;
    }
  }
  free(v);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Stochastic rounding of MXFP4 gradient packs.                           */
/* [P3 Overview, configuration table]: the MXFP4 recipe has one numerics  */
/* switch, stochastic rounding (SR) of the FP4 quantization of gradients. */
/* The page gives neither the rounding rule nor the random source; the    */
/* readings taken here:                                                   */
/*  - the block scale is the FLOOR scale of round-to-nearest packing;     */
/*  - v = x * 2^-X is exact; |v| >= 6 saturates to 6 (no SR there);       */
/*    otherwise with grid neighbours lo <= |v| < hi and                   */
/*    t = (|v| - lo) / (hi - lo), the magnitude is hi iff                 */
/*    (r >> 8) < floor(t * 2^24), for a 32-bit random word r, else lo;    */
/*    the sign is kept (-0 included).  E[result] = v up to 2^-24 of the   */
/*    grid spacing, and values on the grid never move;                    */
/*  - r is a word of Philox4x32-10 (Salmon, Moraes, Dror and Shaw,         */
/*    "Parallel random numbers: as easy as 1, 2, 3", SC 2011), keyed by   */
/*    the 64-bit seed (low word first) with counter                        */
/*    (q mod 2^32, q div 2^32, axis, 0), q = i div 4, where i is the      */
/*    element's index in its packed operand, i = (batch entry * rows +    */
/*    operand row) * K + k, and axis is 0 for the rowwise operand and 1    */
/*    for the columnwise one; the element takes output word i mod 4.      */
/* ------------------------------------------------------------------ */

/* Philox4x32 with 10 rounds.  One round: the two 32x32 -> 64-bit products
 * of counter words 0 and 2 with the round multipliers, counter words
 * recombined as (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,
 * lo(M0*c0)); the key is bumped by the Weyl constants between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t p0 = M0 * (uint64_t)c0, p1 = M1 * (uint64_t)c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The random word of element i of a packed operand (see above). */
uint32_t orc_sr_word(uint64_t seed, int axis, uint64_t i) {
  uint64_t q = i / 4;
  uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), (uint32_t)axis, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[i % 4];
}

/* E2M1 code of the exact value v with the random word r (rule above). */
unsigned orc_encode_e2m1_sr(double v, uint32_t r) {
  unsigned sign = signbit(v) ? 0x8u : 0u;
  double a = fabs(v);
  if (a >= 6.0) return sign | 7u;
  double lo, hi;
  unsigned clo; /* code of lo: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 are codes 0..7 */
  if (a < 2.0) {
    clo = (unsigned)floor(a * 2.0);
    lo = 0.5 * clo;
    hi = lo + 0.5;
  } else if (a < 4.0) {
    lo = floor(a);
    hi = lo + 1.0;
    clo = 4u + (unsigned)(lo - 2.0);
  } else {
    lo = 4.0;
    hi = 6.0;
    clo = 6u;
  }
  double t = (a - lo) / (hi - lo); /* exact: a has 24 significant bits */
  uint64_t k = (uint64_t)floor(t * 16777216.0);
  return sign | (clo + ((uint64_t)(r >> 8) < k ? 1u : 0u));
}

static void quant_block_sr(const float* v, uint64_t seed, int axis, uint64_t i0, unsigned* codes,
                           unsigned* scale) {
  float amax = 0.0f;
  int has_nan = 0;
  for (int i = 0; i < 32; ++i) {
    if (isnan(v[i])) has_nan = 1;
    float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  if (has_nan) amax = NAN;
  unsigned s = orc_scale_floor(ORC_E2M1, amax);
  *scale = s;
  if (s == 0xffu) {
    for (int i = 0; i < 32; ++i) codes[i] = 0u;
    return;
  }
  int e = (int)s - 127;
  for (int i = 0; i < 32; ++i)
    codes[i] = orc_encode_e2m1_sr(ldexp((double)v[i], -e), orc_sr_word(seed, axis, i0 + (uint64_t)i));
}

/* MXFP4 (E2M1, FLOOR scale) pack of the bf16 tensor x [R][C] with
 * stochastic rounding, rowwise ([R] x K=C) and/or columnwise ([C] x K=R,
 * transposed); index_base = batch entry * R * C (the operand index of its
 * first element).  NULL outputs are skipped. */
int orc_quantize_sr(const uint16_t* x, int64_t R, int64_t C, uint64_t seed, uint64_t index_base,
                    uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales) {
  if (R % 32 || C % 32 || R < 0 || C < 0) return 1;
  int64_t rb = orc_row_bytes(ORC_E2M1, C), cb = orc_row_bytes(ORC_E2M1, R);
  if (row_codes) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
      for (int64_t b = 0; b < C / 32; ++b) {
        float blk[32];
        unsigned codes[32], s;
        for (int i = 0; i < 32; ++i) blk[i] = orc_bf16_to_f32(x[r * C + b * 32 + i]);
        quant_block_sr(blk, seed, 0, index_base + (uint64_t)(r * C + b * 32), codes, &s);
        row_scales[r * (C / 32) + b] = (uint8_t)s;
        for (int i = 0; i < 32; ++i) orc_put_code(row_codes + r * rb, ORC_E2M1, b * 32 + i, codes[i]);
      }
    }
  }
  if (col_codes) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
      for (int64_t b = 0; b < R / 32; ++b) {
        float blk[32];
        unsigned codes[32], s;
        for (int i = 0; i < 32; ++i) blk[i] = orc_bf16_to_f32(x[(b * 32 + i) * C + c]);
        quant_block_sr(blk, seed, 1, index_base + (uint64_t)(c * R + b * 32), codes, &s);
        col_scales[c * (R / 32) + b] = (uint8_t)s;
        for (int i = 0; i < 32; ++i) orc_put_code(col_codes + c * cb, ORC_E2M1, b * 32 + i, codes[i]);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Block-scaled GEMM, C = A . B^T (NT layout [P3 Troubleshooting]).       */
/* Both operands are K-major packed codes + [rows][K/32] scales.          */
/* Dequantized values code * 2^(scale-127) are exact in binary64; the     */
/* dot products are summed in binary64 in increasing k; the optional      */
/* bias (bf16 [N]) is added after the full sum [P1 commit messages: the   */
/* bias joins the accumulator and the result is rounded once].  The       */
/* output is binary64, unrounded: callers compare within a tolerance.     */
/* rows: optional list of nrows A-row indices (NULL = all M rows, in     */
/* order); out is [nrows][N].                                              */
/* ------------------------------------------------------------------ */

static double deq(const uint8_t* codes_row, const uint8_t* scales_row, int fmt, int64_t k) {
  unsigned s = scales_row[k / 32];
  double v = orc_decode(fmt, orc_get_code(codes_row, fmt, k));
  if (s == 0xffu) return NAN;
  return ldexp(v, (int)s - 127);
}

int orc_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
             const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, int fmt, const uint16_t* bias,
             const int64_t* rows, int64_t nrows, double* out) {
  if (K % 32) return 1;
  int64_t rb = orc_row_bytes(fmt, K), sb = K / 32;
  /* B dequantized once, stored transposed [K][N] so the inner loop runs over n. */
  double* bt = (double*)malloc((size_t)(K * N > 0 ? K * N : 1) * sizeof(double));
  if (!bt) return 3;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) bt[k * N + n] = deq(b_codes + n * rb, b_scales + n * sb, fmt, k);
  int64_t cnt = rows ? nrows : M;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t i = 0; i < cnt; ++i) {
    int64_t m = rows ? rows[i] : i;
    if (m < 0 || m >= M) { err = 2; continue; }
    double* acc = out + i * N;
    for (int64_t n = 0; n < N; ++n) acc[n] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double a = deq(a_codes + m * rb, a_scales + m * sb, fmt, k);
      const double* brow = bt + k * N;
      for (int64_t n = 0; n < N; ++n) acc[n] = acc[n] + a * brow[n];
    }
    if (bias)
      for (int64_t n = 0; n < N; ++n) acc[n] = acc[n] + (double)orc_bf16_to_f32(bias[n]);
  }
  free(bt);
  return err;
}
