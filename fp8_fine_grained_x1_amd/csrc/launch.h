// Internal interface between the C ABI (abi.cpp) and the kernel files.
// Arguments reaching these launchers have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8fg {

// Compute units of the current device (cached per device).
int device_cu_count();

struct RowtileArgs {
  const void* x;
  int x_type;          // 0 bf16, 1 f32
  int64_t rows, cols, ldx;
  int rule;            // 0 amax, 1 pow2
  uint8_t* q;
  int64_t ldq;
  float* s;
  int64_t s_rs, s_ts;
};
hipError_t launch_quant_1x128(const RowtileArgs& a, hipStream_t st);

// 128 x 128 work blocks: the 128x1 (per-column) and the 128x128 (per-block)
// quantizers, with or without a transposed byte layout.
struct Tile128Args {
  const void* x;
  int x_type;          // 0 bf16, 1 f32, 2 e4m3 (requantization)
  int64_t rows, cols, ldx;
  const float* xs;     // input 1x128 scales (e4m3 input only)
  int64_t xs_rs, xs_ts;
  int rule;
  bool per_column;     // true: 128x1 tiles; false: 128x128 blocks
  bool transpose;      // write q[c * ldq + r]
  uint8_t* q;
  int64_t ldq;
  float* s;
  int64_t s_a, s_b;    // per_column: s[c * s_a + (r/128) * s_b]; block: s[(r/128) * s_a + (c/128) * s_b]
};
hipError_t launch_quant_tile128(const Tile128Args& a, hipStream_t st);

struct GemmArgs {
  int64_t M, N, K;
  const uint8_t* a;
  int64_t lda;
  const float* sa;
  int64_t sa_ms, sa_ks;
  const uint8_t* b;
  int64_t ldb;
  const float* sb;
  int64_t sb_ns, sb_ks;
  int b_scale_mode;    // 0 block128, 1 per column
  void* c;
  int c_type;          // 0 bf16, 1 f32
  int64_t ldc;
  int flags;           // FP8FG_GEMM_* bit set
  // grouped
  int64_t G;           // 0 = dense
  const int32_t* offsets;
  int64_t b_gs, sb_gs;
};
// Which GEMM kernel runs, and its launches (at most two: the default path's
// 256- and 192-column tiles).  Computed on the host from the arguments alone
// (and the CU count), before anything is enqueued, so that the caller can
// check the grid sizes of exactly the launches that will be made.
enum class GemmKernel { kNone, kMx, kStream, kRescale, kBlockscaled };
struct GemmLaunch {
  int64_t tiles_n;   // column tiles of this launch
  int64_t n_base;    // first output column of this launch's tiles
  int64_t nblocks;   // workgroups (0: no launch)
};
struct GemmPlan {
  GemmKernel kernel;
  int mode;          // arithmetic of gemm_blockscaled_kernel (exact / FP8 flags)
  int threads;       // per workgroup
  GemmLaunch launch[2];
};
GemmPlan plan_gemm(const GemmArgs& g, int cus);
hipError_t launch_gemm(const GemmArgs& g, const GemmPlan& plan, hipStream_t st);
// Split of N into column tiles of 256 and 192 for the default GEMM path
// (both zero: the path does not apply).  cus = 0 asks for 256-column tiles
// only (grouped GEMM).
struct ColumnPlan {
  int64_t n256, n192;
};
ColumnPlan plan_columns(int64_t tiles_m, int64_t N, int cus);

}  // namespace fp8fg
