// C ABI of libfp8fg.so: argument validation, then kernel launch.
//
// Every check here runs on the host before any HIP call, so invalid calls
// return an error without touching a device (and can be exercised on a
// machine without a GPU).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fp8fg.h"
#include "launch.h"

namespace fp8fg {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace fp8fg

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_size(int t) { return t == FP8FG_F32 ? 4 : (t == FP8FG_BF16 ? 2 : 1); }

int launched(hipError_t e) { return e == hipSuccess ? FP8FG_OK : FP8FG_ELAUNCH; }

// grids of the 128x128-block quantizers: one 256-thread workgroup per block
constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxGridX = 0xFFFFFFFFll / 256;

}  // namespace

namespace {

constexpr int64_t kMaxPitchA = (int64_t)1 << 23;          // bytes per row of A
constexpr int64_t kMaxPitchB = (int64_t)1 << 24;          // bytes per row of B
constexpr int64_t kMaxScaleRowStride = (int64_t)1 << 21;  // elements
constexpr int64_t kMaxScaleKSpan = (int64_t)1 << 29;      // elements

int check_gemm_common(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                      const float* sa, int64_t sa_ms, int64_t sa_ks, const uint8_t* b,
                      int64_t ldb, const float* sb, int64_t sb_ns, int64_t sb_ks,
                      int b_scale_mode, void* c, int c_type, int64_t ldc, int flags) {
  if (b_scale_mode != FP8FG_BSCALE_BLOCK128 && b_scale_mode != FP8FG_BSCALE_COL) return FP8FG_EINVAL;
  if (c_type != FP8FG_BF16 && c_type != FP8FG_F32) return FP8FG_EINVAL;
  constexpr int kFp8Flags = FP8FG_GEMM_NO_PROMOTION | FP8FG_GEMM_FP8_MFMA | FP8FG_GEMM_E8M0_SCALES;
  constexpr int kTileFlags = FP8FG_GEMM_TILES_WIDE | FP8FG_GEMM_TILES_NARROW;
  if (flags & ~(kFp8Flags | kTileFlags)) return FP8FG_EINVAL;
  if ((flags & FP8FG_GEMM_E8M0_SCALES) && (flags & FP8FG_GEMM_NO_PROMOTION)) return FP8FG_EINVAL;
  // a tile choice exists only on the default path with block scales
  if ((flags & kTileFlags) == kTileFlags) return FP8FG_EINVAL;
  if ((flags & kTileFlags) && ((flags & kFp8Flags) || b_scale_mode != FP8FG_BSCALE_BLOCK128))
    return FP8FG_EINVAL;
  if (M < 0 || N < 0 || K < 0 || lda < 0 || ldb < 0 || ldc < 0) return FP8FG_EINVAL;
  if (sa_ms < 0 || sa_ks < 0 || sb_ns < 0 || sb_ks < 0) return FP8FG_EINVAL;
  if ((flags & FP8FG_GEMM_NO_PROMOTION) && (sa_ks != 0 || sb_ks != 0)) return FP8FG_EINVAL;
  if (K % 128 || N % 128) return FP8FG_ESHAPE;
  if (M == 0 || N == 0) return FP8FG_OK;
  if (!c || !sa || !sb || (K > 0 && (!a || !b))) return FP8FG_EINVAL;
  if (lda < K || ldb < K || ldc < N) return FP8FG_ESHAPE;
  if (!aligned(a, 16) || !aligned(b, 16) || lda % 16 || ldb % 16 ||
      !aligned(c, c_type == FP8FG_F32 ? 4 : 2) || !aligned(sa, 4) || !aligned(sb, 4))
    return FP8FG_EALIGN;
  // The kernels address a tile's operands and scales with 32-bit buffer
  // offsets (row pitch times tile rows, K offsets, scale strides).
  const int64_t nkb = K / 128;
  if (lda >= kMaxPitchA || ldb >= kMaxPitchB || K >= ((int64_t)1 << 31)) return FP8FG_EUNSUPPORTED;
  if (!(flags & FP8FG_GEMM_NO_PROMOTION)) {
    const int64_t kspan = kMaxScaleKSpan / (nkb > 0 ? nkb : 1);
    if (sa_ms >= kMaxScaleRowStride || sa_ks >= kspan || sb_ks >= kspan)
      return FP8FG_EUNSUPPORTED;
    if (b_scale_mode == FP8FG_BSCALE_COL && sb_ns >= kMaxScaleRowStride) return FP8FG_EUNSUPPORTED;
  }
  return FP8FG_OK;
}

// HIP takes at most 2^32 - 1 work-items along a grid dimension.
constexpr int64_t kMaxGridItems = 0xFFFFFFFFll;

// Every launch the plan makes fits the grid limit for its workgroup size.
bool grid_fits(const fp8fg::GemmPlan& pl) {
  for (const fp8fg::GemmLaunch& l : pl.launch)
    if (l.nblocks > kMaxGridItems / pl.threads) return false;
  return true;
}

}  // namespace

extern "C" {

const char* fp8fg_status_string(int status) {
  switch (status) {
    case FP8FG_OK: return "ok";
    case FP8FG_EINVAL: return "invalid argument (null pointer, negative size or stride, bad enum)";
    case FP8FG_ESHAPE: return "bad shape (size not a required multiple of 128, or leading dimension too small)";
    case FP8FG_EALIGN: return "misaligned pointer or row pitch (16-byte alignment required)";
    case FP8FG_EUNSUPPORTED: return "valid but unsupported combination";
    case FP8FG_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int fp8_quantize_rowtile(const void* x, int x_type, int64_t rows, int64_t cols, int64_t ldx,
                         const float* x_scale, int64_t xs_rs, int64_t xs_ts, int tile,
                         int scale_rule, uint8_t* q, int64_t ldq, float* s, int64_t s_rs,
                         int64_t s_ts, void* stream) {
  if (x_type != FP8FG_BF16 && x_type != FP8FG_F32 && x_type != FP8FG_E4M3) return FP8FG_EINVAL;
  if (tile != FP8FG_TILE_1x128 && tile != FP8FG_TILE_128x1) return FP8FG_EINVAL;
  if (scale_rule != FP8FG_SCALE_AMAX && scale_rule != FP8FG_SCALE_POW2) return FP8FG_EINVAL;
  if (rows < 0 || cols < 0 || ldx < 0 || ldq < 0 || s_rs < 0 || s_ts < 0) return FP8FG_EINVAL;
  if (x_type == FP8FG_E4M3 && (xs_rs < 0 || xs_ts < 0)) return FP8FG_EINVAL;
  if (x_type == FP8FG_E4M3 && tile != FP8FG_TILE_128x1) return FP8FG_EUNSUPPORTED;
  if (tile == FP8FG_TILE_1x128) {
    if (cols % 128) return FP8FG_ESHAPE;
  } else {
    if (rows % 128 || cols % 128) return FP8FG_ESHAPE;
  }
  if (rows == 0 || cols == 0) return FP8FG_OK;
  if (!x || !q || !s) return FP8FG_EINVAL;
  if (x_type == FP8FG_E4M3 && !x_scale) return FP8FG_EINVAL;
  if (ldx < cols) return FP8FG_ESHAPE;
  if (ldq < (tile == FP8FG_TILE_1x128 ? cols : rows)) return FP8FG_ESHAPE;
  if (!aligned(x, 16) || (ldx * elem_size(x_type)) % 16 || !aligned(q, 16) || ldq % 16 ||
      !aligned(s, 4) || (x_scale && !aligned(x_scale, 4)))
    return FP8FG_EALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (tile == FP8FG_TILE_1x128) {
    if (rows * (cols / 128) > (int64_t)1 << 31) return FP8FG_EUNSUPPORTED;
    fp8fg::RowtileArgs a{x, x_type, rows, cols, ldx, scale_rule, q, ldq, s, s_rs, s_ts};
    return launched(fp8fg::launch_quant_1x128(a, st));
  }
  if (rows / 128 > kMaxGridY || cols / 128 > kMaxGridX) return FP8FG_EUNSUPPORTED;
  fp8fg::Tile128Args a{x,     x_type, rows, cols, ldx, x_scale, xs_rs, xs_ts, scale_rule,
                       /*per_column=*/true, /*transpose=*/true, q, ldq, s, s_rs, s_ts};
  return launched(fp8fg::launch_quant_tile128(a, st));
}

int fp8_quantize_block(const void* w, int w_type, int64_t rows, int64_t cols, int64_t ldw,
                       int scale_rule, int transpose_out, uint8_t* q, int64_t ldq, float* s,
                       int64_t s_rs, int64_t s_cs, void* stream) {
  if (w_type != FP8FG_BF16 && w_type != FP8FG_F32) return FP8FG_EINVAL;
  if (scale_rule != FP8FG_SCALE_AMAX && scale_rule != FP8FG_SCALE_POW2) return FP8FG_EINVAL;
  if (transpose_out != 0 && transpose_out != 1) return FP8FG_EINVAL;
  if (rows < 0 || cols < 0 || ldw < 0 || ldq < 0 || s_rs < 0 || s_cs < 0) return FP8FG_EINVAL;
  if (rows % 128 || cols % 128) return FP8FG_ESHAPE;
  if (rows == 0 || cols == 0) return FP8FG_OK;
  if (!w || !q || !s) return FP8FG_EINVAL;
  if (ldw < cols || ldq < (transpose_out ? rows : cols)) return FP8FG_ESHAPE;
  if (!aligned(w, 16) || (ldw * elem_size(w_type)) % 16 || !aligned(q, 16) || ldq % 16 ||
      !aligned(s, 4))
    return FP8FG_EALIGN;
  if (rows / 128 > kMaxGridY || cols / 128 > kMaxGridX) return FP8FG_EUNSUPPORTED;
  fp8fg::Tile128Args a{w,       w_type, rows, cols,       ldw,
                       nullptr, 0,      0,    scale_rule, /*per_column=*/false,
                       transpose_out != 0, q, ldq, s, s_rs, s_cs};
  return launched(fp8fg::launch_quant_tile128(a, reinterpret_cast<hipStream_t>(stream)));
}


int fp8_gemm_blockscaled(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                         const float* sa, int64_t sa_ms, int64_t sa_ks, const uint8_t* b,
                         int64_t ldb, const float* sb, int64_t sb_ns, int64_t sb_ks,
                         int b_scale_mode, void* c, int c_type, int64_t ldc, int flags,
                         void* stream) {
  const int rc = check_gemm_common(M, N, K, a, lda, sa, sa_ms, sa_ks, b, ldb, sb, sb_ns, sb_ks,
                                   b_scale_mode, c, c_type, ldc, flags);
  if (rc != FP8FG_OK || M == 0 || N == 0) return rc;
  fp8fg::GemmArgs g{M,  N,  K,  a,      lda,    sa, sa_ms,
                    sa_ks, b, ldb, sb, sb_ns, sb_ks, b_scale_mode,
                    c,  c_type, ldc, flags,
                    0,  nullptr, 0,  0};
  const fp8fg::GemmPlan plan = fp8fg::plan_gemm(g, fp8fg::device_cu_count());
  if (!grid_fits(plan)) return FP8FG_EUNSUPPORTED;
  return launched(fp8fg::launch_gemm(g, plan, reinterpret_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm_blockscaled(int64_t G, const int32_t* offsets, int64_t M_total, int64_t N,
                                 int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                                 int64_t sa_ms, int64_t sa_ks, const uint8_t* b, int64_t ldb,
                                 int64_t b_gs, const float* sb, int64_t sb_ns, int64_t sb_ks,
                                 int64_t sb_gs, void* c, int c_type, int64_t ldc, int flags,
                                 void* stream) {
  if (G < 0 || M_total < 0 || b_gs < 0 || sb_gs < 0) return FP8FG_EINVAL;
  if (G == 0) return M_total == 0 ? FP8FG_OK : FP8FG_EINVAL;
  // the expert offsets are int32, so every row index must be one
  if (G > 0x7FFFFFFF || M_total > 0x7FFFFFFF) return FP8FG_EUNSUPPORTED;
  const int rc = check_gemm_common(M_total, N, K, a, lda, sa, sa_ms, sa_ks, b, ldb, sb, sb_ns,
                                   sb_ks, FP8FG_BSCALE_BLOCK128, c, c_type, ldc, flags);
  if (rc != FP8FG_OK || M_total == 0 || N == 0) return rc;
  if (!offsets) return FP8FG_EINVAL;
  if (!aligned(offsets, 4)) return FP8FG_EALIGN;
  if (b_gs % 16) return FP8FG_EALIGN;
  fp8fg::GemmArgs g{M_total, N,  K,  a,      lda,    sa, sa_ms,
                    sa_ks,   b,  ldb, sb, sb_ns, sb_ks, FP8FG_BSCALE_BLOCK128,
                    c,       c_type, ldc, flags,
                    G,       offsets, b_gs, sb_gs};
  const fp8fg::GemmPlan plan = fp8fg::plan_gemm(g, fp8fg::device_cu_count());
  if (!grid_fits(plan)) return FP8FG_EUNSUPPORTED;
  return launched(fp8fg::launch_gemm(g, plan, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
