// C ABI of libmx: host-side argument validation and launch composition.
// Declarations and the contract of every entry point are in include/mx.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>
#include <vector>

#include "mx.h"
#include "mx_kernels.h"

namespace {

using mx::GemmParams;
using mx::PackParams;

// ---------------------------------------------------------------- helpers
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int bits_of(int fmt) { return fmt == MX_E2M1 ? 4 : fmt == MX_E2M3 ? 6 : fmt == MX_E4M3 ? 8 : 0; }

// Formats, scale modes and rotation the kernels serve: FLOOR for every
// format (E4M3 with FLOOR takes emax 8), RCEIL only with E4M3 (its 448 is
// E4M3's largest value), the rotation only with E2M3.
bool combo_ok(int fmt, int mode, int had) {
  if (bits_of(fmt) == 0) return false;
  if (mode != MX_SCALE_FLOOR && mode != MX_SCALE_RCEIL) return false;
  if (had != 0 && had != 1) return false;
  if (mode == MX_SCALE_RCEIL && fmt != MX_E4M3) return false;
  if (had && fmt != MX_E2M3) return false;
  return true;
}

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int device_state(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 2;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 2;
    g_dev_state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  return g_dev_state[dev];
}

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return MX_ERR_DEVICE;
  }
  return device_state(dev) == 1 ? MX_OK : MX_ERR_DEVICE;
}

int launched(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MX_ERR_LAUNCH;
  }
  return MX_OK;
}

// grid dimensions the launches need must fit
bool grid_fits(int64_t x, int64_t y, int64_t z) {
  return x >= 0 && y >= 0 && z >= 0 && x < (1ll << 31) && y <= 65535 * 1024ll && z <= 65535;
}

// the GEMM kernels address an operand with 32-bit byte offsets
constexpr int64_t kMaxOperandBytes = (1ll << 31) - 1;
bool operand_fits(int fmt, int64_t rows, int64_t k) {
  return rows * (k * bits_of(fmt) / 8) <= kMaxOperandBytes;
}

// ---------------------------------------------------------------- quantize
int validate_quantize(const void* x, const void* aux, int64_t batch, int64_t R, int64_t C, int fmt, int mode,
                      int had, int pro, const void* rc, const void* rs, const void* cc, const void* cs,
                      const float* part, const float* sum) {
  if (!x) return MX_ERR_NULL;
  if ((rc == nullptr) != (rs == nullptr) || (cc == nullptr) != (cs == nullptr)) return MX_ERR_NULL;
  if (!rc && !cc && !part) return MX_ERR_NULL;
  if (sum && !part) return MX_ERR_NULL;
  if (pro < MX_PRO_IDENTITY || pro > MX_PRO_DSWIGLU) return MX_ERR_FORMAT;
  const bool need_aux = (pro == MX_PRO_DGELU_TANH || pro == MX_PRO_DSWIGLU);
  if (need_aux && !aux) return MX_ERR_NULL;
  if (!combo_ok(fmt, mode, had)) return MX_ERR_FORMAT;
  if (batch < 1 || R < 0 || C < 0 || R % 32 || C % 32) return MX_ERR_SHAPE;
  if (pro == MX_PRO_DSWIGLU && C % 64) return MX_ERR_SHAPE;
  const void* ptrs[] = {x, aux, rc, rs, cc, cs, part, sum};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MX_ERR_ALIGN;
  if (!grid_fits((C + 127) / 128, (R + 127) / 128, batch)) return MX_ERR_INDEX_OVERFLOW;
  return MX_OK;
}

int quantize_launch(const void* x, const void* aux, int64_t batch, int64_t R, int64_t C, int fmt, int mode,
                    int had, int pro, void* rc, void* rs, void* cc, void* cs, float* part, float* sum,
                    hipStream_t s) {
  if (R == 0 || C == 0) return MX_OK;
  PackParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.aux = static_cast<const uint16_t*>(aux);
  p.R = R;
  p.C = C;
  p.row_codes = static_cast<uint8_t*>(rc);
  p.row_scales = static_cast<uint8_t*>(rs);
  p.col_codes = static_cast<uint8_t*>(cc);
  p.col_scales = static_cast<uint8_t*>(cs);
  p.partials = part;
  p.sr_seed = 0;
  int st = launched(mx::launch_pack(p, fmt, mode, had, pro, batch, s));
  if (st != MX_OK) return st;
  if (sum) st = launched(mx::launch_colsum_finish(part, R / 32, C, sum, batch, s));
  return st;
}

// ---------------------------------------------------------------- GEMM
int validate_gemm(const void* ac, const void* as, const void* bc, const void* bs, int64_t M, int64_t N,
                  int64_t K, int fmt, const void* bias, int bias_dtype, const void* c, int c_dtype, int64_t ldc) {
  if (!ac || !as || !bc || !bs || !c) return MX_ERR_NULL;
  if (bits_of(fmt) == 0) return MX_ERR_FORMAT;
  if ((bias_dtype != MX_BF16 && bias_dtype != MX_F32) || (c_dtype != MX_BF16 && c_dtype != MX_F32))
    return MX_ERR_FORMAT;
  if (M < 0 || N < 0 || K < 0 || M % 256 || N % 256 || K % 256) return MX_ERR_SHAPE;
  if (ldc < N || ldc % 8) return MX_ERR_SHAPE;
  const void* ptrs[] = {ac, as, bc, bs, bias, c};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MX_ERR_ALIGN;
  // the dense launch's 1-D grid of output tiles (none is smaller than 128 x 128)
  if (!grid_fits((M / 128) * (N / 128), 1, 1)) return MX_ERR_INDEX_OVERFLOW;
  if (!operand_fits(fmt, M, K) || !operand_fits(fmt, N, K)) return MX_ERR_INDEX_OVERFLOW;
  return MX_OK;
}

int gemm_launch(const void* ac, const void* as, const void* bc, const void* bs, int64_t M, int64_t N, int64_t K,
                int fmt, const void* bias, int bias_dtype, void* c, int c_dtype, int64_t ldc, int accumulate,
                hipStream_t s, int tile_shape = 0) {
  if (M == 0 || N == 0) return MX_OK;
  GemmParams p;
  memset(&p, 0, sizeof p);
  p.a_codes = static_cast<const uint8_t*>(ac);
  p.a_scales = static_cast<const uint8_t*>(as);
  p.b_codes = static_cast<const uint8_t*>(bc);
  p.b_scales = static_cast<const uint8_t*>(bs);
  p.M = M;
  p.N = N;
  p.K = K;
  p.ktot = K;
  p.bias = bias;
  p.bias_f32 = bias_dtype == MX_F32;
  p.c = c;
  p.ldc = ldc;
  p.c_f32 = c_dtype == MX_F32;
  p.tile_shape = tile_shape;
  return launched(mx::launch_gemm(p, fmt, mx::kDense, accumulate ? mx::kEpiAccum : mx::kEpiStore, s));
}

// ---------------------------------------------------------------- static scratch
// The work buffer of mx_quantize_noalloc: one copy per GPU, allocated with
// the code object and kept until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: the device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kernels.
static_assert(MX_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[MX_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, or nullptr until looked up

// Device address of the current device's scratch array (looked up on the
// first call on that device), or nullptr if the runtime cannot give it.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Shader clock over a wall-clock interval: one wavefront reads the shader
// cycle counter (s_memtime) and the constant-rate wall clock (s_memrealtime)
// before and after spinning until `wall_ticks` wall-clock ticks have passed
// (a bounded wait: the wall clock always advances).  out[0] = shader
// cycles, out[1] = wall-clock ticks.
__global__ __launch_bounds__(64) void clock_sample_kernel(uint64_t wall_ticks, uint64_t* out) {
  const uint64_t r0 = wall_clock64(), c0 = clock64();
  uint64_t r1 = r0;
  while (r1 - r0 < wall_ticks) r1 = wall_clock64();
  const uint64_t c1 = clock64();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

bool packed_ok(const mx_packed& q) { return q.codes && q.scales; }
bool packed_aligned(const mx_packed& q) { return aligned16(q.codes) && aligned16(q.scales); }

}  // namespace

extern "C" {

int mx_quantize(const void* x, const void* aux, int64_t batch, int64_t R, int64_t C, int fmt, int scale_mode,
                int hadamard, int prologue, void* row_codes, void* row_scales, void* col_codes, void* col_scales,
                float* colsum_partials, float* colsum, void* stream) {
  int st = validate_quantize(x, aux, batch, R, C, fmt, scale_mode, hadamard, prologue, row_codes, row_scales,
                             col_codes, col_scales, colsum_partials, colsum);
  if (st != MX_OK) return st;
  if ((st = check_device()) != MX_OK) return st;
  return quantize_launch(x, aux, batch, R, C, fmt, scale_mode, hadamard, prologue, row_codes, row_scales,
                         col_codes, col_scales, colsum_partials, colsum, static_cast<hipStream_t>(stream));
}

int mx_quantize_noalloc(const void* x, const void* aux, int64_t batch, int64_t R, int64_t C, int fmt,
                        int scale_mode, int hadamard, int prologue, void* row_codes, void* row_scales,
                        void* col_codes, void* col_scales, float* colsum, void* stream) {
  // the partials pointer only stands for "present" in the checks below; it
  // is replaced by the scratch address before any launch
  float* const marker = colsum ? colsum : nullptr;
  int st = validate_quantize(x, aux, batch, R, C, fmt, scale_mode, hadamard, prologue, row_codes, row_scales,
                             col_codes, col_scales, marker, colsum);
  if (st != MX_OK) return st;
  if (colsum && (batch * (R / 32) * C > (int64_t)(MX_NOALLOC_SCRATCH_BYTES / sizeof(float))))
    return MX_ERR_SCRATCH;
  if ((st = check_device()) != MX_OK) return st;
  float* part = nullptr;
  if (colsum) {
    part = static_cast<float*>(scratch_ptr());
    if (!part) return MX_ERR_DEVICE;
  }
  return quantize_launch(x, aux, batch, R, C, fmt, scale_mode, hadamard, prologue, row_codes, row_scales,
                         col_codes, col_scales, part, colsum, static_cast<hipStream_t>(stream));
}

int mx_quantize_sr(const void* x, int64_t batch, int64_t R, int64_t C, void* row_codes, void* row_scales,
                   void* col_codes, void* col_scales, float* colsum_partials, float* colsum, uint64_t seed,
                   void* stream) {
  int st = validate_quantize(x, nullptr, batch, R, C, MX_E2M1, MX_SCALE_FLOOR, 0, MX_PRO_IDENTITY, row_codes,
                             row_scales, col_codes, col_scales, colsum_partials, colsum);
  if (st != MX_OK) return st;
  if ((st = check_device()) != MX_OK) return st;
  if (R == 0 || C == 0) return MX_OK;
  PackParams p;
  memset(&p, 0, sizeof p);
  p.x = static_cast<const uint16_t*>(x);
  p.R = R;
  p.C = C;
  p.row_codes = static_cast<uint8_t*>(row_codes);
  p.row_scales = static_cast<uint8_t*>(row_scales);
  p.col_codes = static_cast<uint8_t*>(col_codes);
  p.col_scales = static_cast<uint8_t*>(col_scales);
  p.partials = colsum_partials;
  p.sr_seed = seed;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = launched(mx::launch_pack_sr(p, batch, s))) != MX_OK) return st;
  if (colsum) st = launched(mx::launch_colsum_finish(colsum_partials, R / 32, C, colsum, batch, s));
  return st;
}

int mx_quantize_many(const mx_quantize_item* items, int n, int fmt, int scale_mode, int hadamard, int prologue,
                     void* stream) {
  if (!items) return MX_ERR_NULL;
  if (n < 1 || n > MX_QUANTIZE_MANY_MAX) return MX_ERR_SHAPE;
  static_assert(MX_QUANTIZE_MANY_MAX == mx::kPackManyMax, "item limit");
  mx::PackMany m;
  memset(&m, 0, sizeof m);
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    const mx_quantize_item& it = items[i];
    int st = validate_quantize(it.x, it.aux, it.batch, it.R, it.C, fmt, scale_mode, hadamard, prologue,
                               it.row.codes, it.row.scales, it.col.codes, it.col.scales, it.colsum_partials,
                               it.colsum);
    if (st != MX_OK) return st;
    PackParams& p = m.p[i];
    p.x = static_cast<const uint16_t*>(it.x);
    p.aux = static_cast<const uint16_t*>(it.aux);
    p.R = it.R;
    p.C = it.C;
    p.row_codes = static_cast<uint8_t*>(it.row.codes);
    p.row_scales = static_cast<uint8_t*>(it.row.scales);
    p.col_codes = static_cast<uint8_t*>(it.col.codes);
    p.col_scales = static_cast<uint8_t*>(it.col.scales);
    p.partials = it.colsum_partials;
    m.first[i] = tiles;
    tiles += ((it.C + 127) / 128) * ((it.R + 127) / 128) * it.batch;
  }
  m.first[n] = tiles;
  m.n = n;
  if (!grid_fits(tiles, 1, 1)) return MX_ERR_INDEX_OVERFLOW;
  int st = check_device();
  if (st != MX_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = launched(mx::launch_pack_many(m, fmt, scale_mode, hadamard, prologue, s))) != MX_OK) return st;
  for (int i = 0; i < n; ++i) {
    const mx_quantize_item& it = items[i];
    if (it.colsum && it.R > 0 && it.C > 0)
      if ((st = launched(mx::launch_colsum_finish(it.colsum_partials, it.R / 32, it.C, it.colsum, it.batch, s))) !=
          MX_OK)
        return st;
  }
  return MX_OK;
}

int mx_gemm(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales, int64_t M,
            int64_t N, int64_t K, int fmt, const void* bias, int bias_dtype, void* c, int c_dtype, int64_t ldc,
            void* stream) {
  int st = validate_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias, bias_dtype, c, c_dtype, ldc);
  if (st != MX_OK) return st;
  if ((st = check_device()) != MX_OK) return st;
  return gemm_launch(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias, bias_dtype, c, c_dtype, ldc, 0,
                     static_cast<hipStream_t>(stream));
}

int mx_gemm_accumulate(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales,
                       int64_t M, int64_t N, int64_t K, int fmt, const void* bias, int bias_dtype, void* c,
                       int c_dtype, int64_t ldc, void* stream) {
  int st = validate_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias, bias_dtype, c, c_dtype, ldc);
  if (st != MX_OK) return st;
  if ((st = check_device()) != MX_OK) return st;
  return gemm_launch(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias, bias_dtype, c, c_dtype, ldc, 1,
                     static_cast<hipStream_t>(stream));
}

int mx_gemm_tiled(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales, int64_t M,
                  int64_t N, int64_t K, int fmt, const void* bias, int bias_dtype, void* c, int c_dtype, int64_t ldc,
                  int tile_m, int tile_n, int wg_per_cu, void* stream) {
  int st = validate_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias, bias_dtype, c, c_dtype, ldc);
  if (st != MX_OK) return st;
  int tile = 0;
  if (tile_m != 0 || tile_n != 0 || wg_per_cu != 0) {
    const int i = mx::dense_tile_index(tile_m, tile_n, wg_per_cu, M, N);
    if (i < 0) return MX_ERR_SHAPE;
    tile = i + 1;
  }
  if ((st = check_device()) != MX_OK) return st;
  return gemm_launch(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias, bias_dtype, c, c_dtype, ldc, 0,
                     static_cast<hipStream_t>(stream), tile);
}

int mx_gemm_plan(int64_t M, int64_t N, int64_t K, int fmt, int* plan, int64_t* workspace_bytes) {
  if (!plan) return MX_ERR_NULL;
  if (bits_of(fmt) == 0) return MX_ERR_FORMAT;
  if (M < 0 || N < 0 || K < 0 || M % 256 || N % 256 || K % 256) return MX_ERR_SHAPE;
  mx::GemmPlan g;
  if (!mx::plan_gemm(fmt, M, N, K, &g)) return MX_ERR_SHAPE;
  plan[0] = g.tile_m;
  plan[1] = g.tile_n;
  plan[2] = g.wg_per_cu;
  plan[3] = g.split_k;
  if (workspace_bytes) *workspace_bytes = g.split_k > 1 ? (int64_t)g.split_k * M * N * 4 : 0;
  return MX_OK;
}

int mx_gemm_splitk(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales, int64_t M,
                   int64_t N, int64_t K, int fmt, const void* bias, int bias_dtype, void* c, int c_dtype,
                   int64_t ldc, int tile_m, int tile_n, int wg_per_cu, int split_k, void* workspace,
                   int64_t workspace_bytes, void* stream) {
  int st = validate_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias, bias_dtype, c, c_dtype, ldc);
  if (st != MX_OK) return st;
  if (split_k < 1 || split_k > MX_SPLIT_K_MAX || K % (128 * (int64_t)split_k)) return MX_ERR_SHAPE;
  int tile = 0;
  if (tile_m != 0 || tile_n != 0 || wg_per_cu != 0) {
    const int i = mx::dense_tile_index(tile_m, tile_n, wg_per_cu, M, N);
    if (i < 0) return MX_ERR_SHAPE;
    tile = i + 1;
  }
  if (split_k > 1) {
    if (!workspace) return MX_ERR_NULL;
    if (!aligned16(workspace)) return MX_ERR_ALIGN;
    if (workspace_bytes < (int64_t)split_k * M * N * 4) return MX_ERR_SHAPE;
    if (!grid_fits((M / 128) * (N / 128) * split_k, 1, 1) || !grid_fits(M * (N / 4) / 256 + 1, 1, 1))
      return MX_ERR_INDEX_OVERFLOW;
  }
  if ((st = check_device()) != MX_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (split_k == 1)
    return gemm_launch(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt, bias, bias_dtype, c, c_dtype, ldc, 0, s,
                       tile);
  if (M == 0 || N == 0) return MX_OK;
  GemmParams p;
  memset(&p, 0, sizeof p);
  p.a_codes = static_cast<const uint8_t*>(a_codes);
  p.a_scales = static_cast<const uint8_t*>(a_scales);
  p.b_codes = static_cast<const uint8_t*>(b_codes);
  p.b_scales = static_cast<const uint8_t*>(b_scales);
  p.M = M;
  p.N = N;
  p.K = K;
  p.ktot = K;
  p.c = workspace;  // part s at workspace + s * M * N, binary32, no bias
  p.ldc = N;
  p.c_f32 = 1;
  p.tile_shape = tile;
  p.split_k = split_k;
  if ((st = launched(mx::launch_gemm(p, fmt, mx::kDense, mx::kEpiSplit, s))) != MX_OK) return st;
  return launched(mx::launch_splitk_reduce(static_cast<const float*>(workspace), split_k, M, N, bias,
                                           bias_dtype == MX_F32, c, c_dtype == MX_F32, ldc, s));
}

int mx_gemm_many(const mx_gemm_item* items, int n, int fmt, void* stream) {
  if (!items) return MX_ERR_NULL;
  if (n < 1 || n > MX_GEMM_MANY_MAX) return MX_ERR_SHAPE;
  static_assert(MX_GEMM_MANY_MAX == mx::kGemmManyMax, "item limit");
  mx::GemmMany m;
  memset(&m, 0, sizeof m);
  for (int i = 0; i < n; ++i) {
    const mx_gemm_item& it = items[i];
    int st = validate_gemm(it.A.codes, it.A.scales, it.B.codes, it.B.scales, it.M, it.N, it.K, fmt, it.bias,
                           it.bias_dtype, it.C, it.c_dtype, it.ldc);
    if (st != MX_OK) return st;
    if (it.accumulate != 0 && it.accumulate != 1) return MX_ERR_FORMAT;
    if (it.M == 0 || it.N == 0 || it.accumulate) continue;  // accumulating items: a launch each, below
    GemmParams& p = m.p[m.n++];
    p.a_codes = static_cast<const uint8_t*>(it.A.codes);
    p.a_scales = static_cast<const uint8_t*>(it.A.scales);
    p.b_codes = static_cast<const uint8_t*>(it.B.codes);
    p.b_scales = static_cast<const uint8_t*>(it.B.scales);
    p.M = it.M;
    p.N = it.N;
    p.K = it.K;
    p.ktot = it.K;
    p.bias = it.bias;
    p.bias_f32 = it.bias_dtype == MX_F32;
    p.c = it.C;
    p.ldc = it.ldc;
    p.c_f32 = it.c_dtype == MX_F32;
  }
  int st = check_device();
  if (st != MX_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (m.n > 0 && (st = launched(mx::launch_gemm_many(m, fmt, s))) != MX_OK) return st;
  for (int i = 0; i < n; ++i) {
    const mx_gemm_item& it = items[i];
    if (!it.accumulate) continue;
    if ((st = gemm_launch(it.A.codes, it.A.scales, it.B.codes, it.B.scales, it.M, it.N, it.K, fmt, it.bias,
                          it.bias_dtype, it.C, it.c_dtype, it.ldc, 1, s)) != MX_OK)
      return st;
  }
  return MX_OK;
}

int mx_fused_mlp_fwd(const mx_mlp_fwd_args* a, void* stream) {
  if (!a) return MX_ERR_NULL;
  if (!a->X || !a->W1 || !a->W2 || !a->h || !a->Y) return MX_ERR_NULL;
  const mx_packed* packs[] = {&a->Xr, &a->Xc, &a->W1r, &a->W1c, &a->W2r, &a->W2c, &a->ar, &a->ac};
  for (const mx_packed* q : packs)
    if (!packed_ok(*q)) return MX_ERR_NULL;
  if (!combo_ok(a->fmt, a->scale_mode, a->hadamard)) return MX_ERR_FORMAT;
  const int64_t M = a->M, D = a->D, F = a->F;
  if (M < 0 || D < 0 || F < 0 || M % 256 || D % 256 || F % 256) return MX_ERR_SHAPE;
  const void* ptrs[] = {a->X, a->W1, a->b1, a->W2, a->h, a->Y};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MX_ERR_ALIGN;
  for (const mx_packed* q : packs)
    if (!packed_aligned(*q)) return MX_ERR_ALIGN;
  const int fmt = a->fmt, mode = a->scale_mode, had = a->hadamard;
  // every pack and GEMM of the composition passes the checks of its own
  // entry point (grid and 32-bit offset limits included)
  int st;
  if ((st = validate_quantize(a->X, nullptr, 1, M, D, fmt, mode, had, MX_PRO_IDENTITY, a->Xr.codes, a->Xr.scales,
                              a->Xc.codes, a->Xc.scales, nullptr, nullptr)) ||
      (st = validate_quantize(a->W1, nullptr, 1, F, D, fmt, mode, had, MX_PRO_IDENTITY, a->W1r.codes,
                              a->W1r.scales, a->W1c.codes, a->W1c.scales, nullptr, nullptr)) ||
      (st = validate_quantize(a->W2, nullptr, 1, D, F, fmt, mode, had, MX_PRO_IDENTITY, a->W2r.codes,
                              a->W2r.scales, a->W2c.codes, a->W2c.scales, nullptr, nullptr)) ||
      (st = validate_quantize(a->h, nullptr, 1, M, F, fmt, mode, had, MX_PRO_GELU_TANH, a->ar.codes, a->ar.scales,
                              a->ac.codes, a->ac.scales, nullptr, nullptr)) ||
      (st = validate_gemm(a->Xr.codes, a->Xr.scales, a->W1r.codes, a->W1r.scales, M, F, D, fmt, a->b1, MX_BF16,
                          a->h, MX_BF16, F)) ||
      (st = validate_gemm(a->ar.codes, a->ar.scales, a->W2r.codes, a->W2r.scales, M, D, F, fmt, nullptr, MX_BF16,
                          a->Y, MX_BF16, D)) ||
      (st = operand_fits(fmt, D, M) && operand_fits(fmt, D, F) && operand_fits(fmt, F, D) && operand_fits(fmt, F, M)
                ? MX_OK
                : MX_ERR_INDEX_OVERFLOW))
    return st;
  if ((st = check_device()) != MX_OK) return st;
  if (M == 0 || D == 0 || F == 0) return MX_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // packs of X, W1, W2 (rows for the forward, columns kept for the
  // backward), in one launch: the same tile body as one launch each, so
  // the same bytes, without two launch boundaries and their drained tails
  {
    mx::PackMany m;
    memset(&m, 0, sizeof m);
    const void* xs[3] = {a->X, a->W1, a->W2};
    const int64_t rs[3] = {M, F, D}, cs[3] = {D, D, F};
    const mx_packed* rows[3] = {&a->Xr, &a->W1r, &a->W2r};
    const mx_packed* cols[3] = {&a->Xc, &a->W1c, &a->W2c};
    int64_t tiles = 0;
    for (int i = 0; i < 3; ++i) {
      PackParams& q = m.p[i];
      q.x = static_cast<const uint16_t*>(xs[i]);
      q.R = rs[i];
      q.C = cs[i];
      q.row_codes = static_cast<uint8_t*>(rows[i]->codes);
      q.row_scales = static_cast<uint8_t*>(rows[i]->scales);
      q.col_codes = static_cast<uint8_t*>(cols[i]->codes);
      q.col_scales = static_cast<uint8_t*>(cols[i]->scales);
      m.first[i] = tiles;
      tiles += ((cs[i] + 127) / 128) * ((rs[i] + 127) / 128);
    }
    m.first[3] = tiles;
    m.n = 3;
    if (!grid_fits(tiles, 1, 1)) return MX_ERR_INDEX_OVERFLOW;
    if ((st = launched(mx::launch_pack_many(m, fmt, mode, had, MX_PRO_IDENTITY, s))) != MX_OK) return st;
  }
  // fc1: h = X W1^T + b1 (bias in the fp32 accumulator, one rounding)
  if ((st = gemm_launch(a->Xr.codes, a->Xr.scales, a->W1r.codes, a->W1r.scales, M, F, D, fmt, a->b1, MX_BF16,
                        a->h, MX_BF16, F, 0, s)))
    return st;
  // a = GELU(h) exists only inside the packer: packed rows for fc2, columns for dW2
  if ((st = quantize_launch(a->h, nullptr, 1, M, F, fmt, mode, had, MX_PRO_GELU_TANH, a->ar.codes, a->ar.scales,
                            a->ac.codes, a->ac.scales, nullptr, nullptr, s)))
    return st;
  // fc2: Y = a W2^T
  return gemm_launch(a->ar.codes, a->ar.scales, a->W2r.codes, a->W2r.scales, M, D, F, fmt, nullptr, MX_BF16, a->Y,
                     MX_BF16, D, 0, s);
}

int mx_fused_mlp_bwd(const mx_mlp_bwd_args* a, void* stream) {
  if (!a) return MX_ERR_NULL;
  if (!a->dY || !a->h || !a->da || !a->dX || !a->dW1 || !a->dW2) return MX_ERR_NULL;
  if (a->db1 && !a->db1_partials) return MX_ERR_NULL;
  const mx_packed* packs[] = {&a->Xc, &a->W1c, &a->W2c, &a->ac, &a->dYr, &a->dYc, &a->dhr, &a->dhc};
  for (const mx_packed* q : packs)
    if (!packed_ok(*q)) return MX_ERR_NULL;
  if (!combo_ok(a->fmt, a->scale_mode, a->hadamard)) return MX_ERR_FORMAT;
  if (a->accumulate_wgrad != 0 && a->accumulate_wgrad != 1) return MX_ERR_FORMAT;
  const int64_t M = a->M, D = a->D, F = a->F;
  if (M < 0 || D < 0 || F < 0 || M % 256 || D % 256 || F % 256) return MX_ERR_SHAPE;
  const void* ptrs[] = {a->dY, a->h, a->da, a->dX, a->dW1, a->dW2, a->db1, a->db1_partials};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MX_ERR_ALIGN;
  for (const mx_packed* q : packs)
    if (!packed_aligned(*q)) return MX_ERR_ALIGN;
  const int fmt = a->fmt, mode = a->scale_mode, had = a->hadamard;
  // every pack and GEMM of the composition passes the checks of its own
  // entry point (grid and 32-bit offset limits included)
  int st;
  float* part = a->db1 ? a->db1_partials : nullptr;
  if ((st = validate_quantize(a->dY, nullptr, 1, M, D, fmt, mode, had, MX_PRO_IDENTITY, a->dYr.codes,
                              a->dYr.scales, a->dYc.codes, a->dYc.scales, nullptr, nullptr)) ||
      (st = validate_quantize(a->da, a->h, 1, M, F, fmt, mode, had, MX_PRO_DGELU_TANH, a->dhr.codes, a->dhr.scales,
                              a->dhc.codes, a->dhc.scales, part, a->db1)) ||
      (st = validate_gemm(a->dYr.codes, a->dYr.scales, a->W2c.codes, a->W2c.scales, M, F, D, fmt, nullptr, MX_BF16,
                          a->da, MX_BF16, F)) ||
      (st = validate_gemm(a->dhr.codes, a->dhr.scales, a->W1c.codes, a->W1c.scales, M, D, F, fmt, nullptr, MX_BF16,
                          a->dX, MX_BF16, D)) ||
      (st = validate_gemm(a->dhc.codes, a->dhc.scales, a->Xc.codes, a->Xc.scales, F, D, M, fmt, nullptr, MX_BF16,
                          a->dW1, MX_BF16, D)) ||
      (st = validate_gemm(a->dYc.codes, a->dYc.scales, a->ac.codes, a->ac.scales, D, F, M, fmt, nullptr, MX_BF16,
                          a->dW2, MX_BF16, F)))
    return st;
  if ((st = check_device()) != MX_OK) return st;
  if (M == 0 || D == 0 || F == 0) return MX_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = quantize_launch(a->dY, nullptr, 1, M, D, fmt, mode, had, MX_PRO_IDENTITY, a->dYr.codes, a->dYr.scales,
                            a->dYc.codes, a->dYc.scales, nullptr, nullptr, s)))
    return st;
  // fc2 dgrad: da = dY W2 (K = D), materialised
  if ((st = gemm_launch(a->dYr.codes, a->dYr.scales, a->W2c.codes, a->W2c.scales, M, F, D, fmt, nullptr, MX_BF16,
                        a->da, MX_BF16, F, 0, s)))
    return st;
  // dh = dGELU(da, h) exists only inside the packer; bias gradient from its column sums
  if ((st = quantize_launch(a->da, a->h, 1, M, F, fmt, mode, had, MX_PRO_DGELU_TANH, a->dhr.codes, a->dhr.scales,
                            a->dhc.codes, a->dhc.scales, a->db1 ? a->db1_partials : nullptr, a->db1, s)))
    return st;
  // fc1 dgrad: dX = dh W1 (K = F)
  if ((st = gemm_launch(a->dhr.codes, a->dhr.scales, a->W1c.codes, a->W1c.scales, M, D, F, fmt, nullptr, MX_BF16,
                        a->dX, MX_BF16, D, 0, s)))
    return st;
  // fc1 wgrad: dW1 = dh^T X (K = M)
  if ((st = gemm_launch(a->dhc.codes, a->dhc.scales, a->Xc.codes, a->Xc.scales, F, D, M, fmt, nullptr, MX_BF16,
                        a->dW1, MX_BF16, D, a->accumulate_wgrad, s)))
    return st;
  // fc2 wgrad: dW2 = dY^T a (K = M)
  return gemm_launch(a->dYc.codes, a->dYc.scales, a->ac.codes, a->ac.scales, D, F, M, fmt, nullptr, MX_BF16,
                     a->dW2, MX_BF16, F, a->accumulate_wgrad, s);
}

int mx_grouped_gemm(const mx_grouped_args* a, void* stream) {
  if (!a) return MX_ERR_NULL;
  if (!a->offsets || !packed_ok(a->A) || !packed_ok(a->B)) return MX_ERR_NULL;
  if (bits_of(a->fmt) == 0) return MX_ERR_FORMAT;
  if (a->mode != MX_GROUPED_RAGGED_M && a->mode != MX_GROUPED_RAGGED_K) return MX_ERR_FORMAT;
  if (a->epilogue < MX_EPI_NONE || a->epilogue > MX_EPI_DSWIGLU) return MX_ERR_FORMAT;
  if (a->mode == MX_GROUPED_RAGGED_K && a->epilogue != MX_EPI_NONE) return MX_ERR_FORMAT;
  const bool quant = a->epilogue != MX_EPI_NONE;
  if (quant) {
    if (!combo_ok(a->fmt, a->scale_mode, 0)) return MX_ERR_FORMAT;
    if (!packed_ok(a->out_row) || !packed_ok(a->out_col)) return MX_ERR_NULL;
    if (a->epilogue == MX_EPI_DSWIGLU && !a->aux) return MX_ERR_NULL;
  }
  if (a->epilogue != MX_EPI_DSWIGLU && !a->C) return MX_ERR_NULL;
  if (a->G < 1 || a->G > 65535 || a->R < 0 || a->R % 128) return MX_ERR_SHAPE;
  if (a->mode == MX_GROUPED_RAGGED_M) {
    if (a->N <= 0 || a->K < 0 || a->N % 256 || a->K % 256) return MX_ERR_SHAPE;
  } else {
    if (a->M < 0 || a->N < 0 || a->M % 256 || a->N % 256) return MX_ERR_SHAPE;
  }
  const void* ptrs[] = {a->offsets, a->A.codes, a->A.scales, a->B.codes, a->B.scales, a->C, a->aux,
                        a->out_row.codes, a->out_row.scales, a->out_col.codes, a->out_col.scales};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MX_ERR_ALIGN;
  if (!grid_fits(a->N / 128 + 1, a->R / 128 + a->M / 128, a->G)) return MX_ERR_INDEX_OVERFLOW;
  if (a->mode == MX_GROUPED_RAGGED_M
          ? (!operand_fits(a->fmt, a->R, a->K) || !operand_fits(a->fmt, (int64_t)a->G * a->N, a->K))
          : (!operand_fits(a->fmt, a->M, a->R) || !operand_fits(a->fmt, a->N, a->R)))
    return MX_ERR_INDEX_OVERFLOW;
  int st = check_device();
  if (st != MX_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->validate_offsets) {
    std::vector<int32_t> off(a->G);
    if (hipMemcpyAsync(off.data(), a->offsets, sizeof(int32_t) * a->G, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
      (void)hipGetLastError();
      return MX_ERR_LAUNCH;
    }
    int32_t prev = 0;
    for (int i = 0; i < a->G; ++i) {
      if (off[i] < prev || off[i] % 128 || off[i] > a->R) return MX_ERR_OFFSETS;
      prev = off[i];
    }
  }
  GemmParams p;
  memset(&p, 0, sizeof p);
  p.a_codes = static_cast<const uint8_t*>(a->A.codes);
  p.a_scales = static_cast<const uint8_t*>(a->A.scales);
  p.b_codes = static_cast<const uint8_t*>(a->B.codes);
  p.b_scales = static_cast<const uint8_t*>(a->B.scales);
  p.offsets = a->offsets;
  p.G = a->G;
  p.R = a->R;
  p.c = a->C;
  p.c_f32 = 0;
  p.q_mode = a->scale_mode;
  if (a->mode == MX_GROUPED_RAGGED_M) {
    if (a->R == 0) return MX_OK;
    p.M = a->R;
    p.N = a->N;
    p.K = a->K;
    p.ktot = a->K;
    p.ldc = a->N;
    p.b_group_rows = a->N;
    p.F = a->epilogue == MX_EPI_SWIGLU ? a->N / 2 : a->N;
    p.aux = static_cast<const uint16_t*>(a->aux);
    p.q_row_codes = static_cast<uint8_t*>(a->out_row.codes);
    p.q_row_scales = static_cast<uint8_t*>(a->out_row.scales);
    p.q_col_codes = static_cast<uint8_t*>(a->out_col.codes);
    p.q_col_scales = static_cast<uint8_t*>(a->out_col.scales);
    const int epi = a->epilogue == MX_EPI_SWIGLU ? mx::kEpiSwiglu
                    : a->epilogue == MX_EPI_DSWIGLU ? mx::kEpiDSwiglu
                                                     : mx::kEpiStore;
    if (epi == mx::kEpiSwiglu && (a->N / 2) % 128) return MX_ERR_SHAPE;
    return launched(mx::launch_gemm(p, a->fmt, mx::kRaggedM, epi, s));
  }
  if (a->M == 0 || a->N == 0) return MX_OK;
  p.M = a->M;
  p.N = a->N;
  p.K = 0;
  p.ktot = a->R;
  p.ldc = a->N;
  return launched(mx::launch_gemm(p, a->fmt, mx::kRaggedK, mx::kEpiStore, s));
}

const char* mx_status_str(int status) {
  switch (status) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: a size is out of range or not the required multiple";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: a device pointer is not 16-byte aligned";
    case MX_ERR_FORMAT: return "MX_ERR_FORMAT: unsupported format / scale mode / prologue / epilogue combination";
    case MX_ERR_OFFSETS: return "MX_ERR_OFFSETS: group offsets break their contract";
    case MX_ERR_INDEX_OVERFLOW: return "MX_ERR_INDEX_OVERFLOW: a size exceeds what one launch can index";
    case MX_ERR_DEVICE: return "MX_ERR_DEVICE: no gfx950 device is current";
    case MX_ERR_LAUNCH: return "MX_ERR_LAUNCH: the HIP runtime failed to enqueue";
    case MX_ERR_SCRATCH: return "MX_ERR_SCRATCH: the call needs more than the library's static scratch holds";
    default: return "unknown mx status";
  }
}

int mx_device_supported(int device) { return device_state(device) == 1 ? 1 : 0; }

int64_t mx_codes_bytes(int fmt, int64_t rows, int64_t K) {
  const int b = bits_of(fmt);
  if (!b || rows < 0 || K < 0 || K % 32) return 0;
  return mx::code_bytes(rows, K, b);
}

int64_t mx_scales_bytes(int64_t rows, int64_t K) {
  if (rows < 0 || K < 0 || K % 32) return 0;
  return mx::scale_bytes(rows, K);
}

const char* mx_version(void) { return "libmx 0.1 (gfx950)"; }

int mx_clock_sample(int64_t microseconds, uint64_t* out, void* stream) {
  if (!out) return MX_ERR_NULL;
  if (!aligned16(out)) return MX_ERR_ALIGN;
  if (microseconds <= 0 || microseconds > 1000000) return MX_ERR_SHAPE;
  int st = check_device();
  if (st != MX_OK) return st;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      khz <= 0) {
    (void)hipGetLastError();
    return MX_ERR_DEVICE;
  }
  const uint64_t ticks = (uint64_t)microseconds * (uint64_t)khz / 1000u;
  hipLaunchKernelGGL(clock_sample_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ticks, out);
  return launched(hipGetLastError());
}

int64_t mx_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return khz;
}

}  // extern "C"
