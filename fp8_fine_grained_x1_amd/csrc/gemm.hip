// Block-scaled FP8 GEMM (dense and grouped) for gfx950.
//
// The method ([thedaegu] Figure 7(b) passage; [fooled] promotion paragraph;
// [hearaon] accumulation-precision paragraph; page keys in
// include/fp8fg.h): an FP8 GEMM whose operands carry one scale per 128
// elements of K sums each 128-wide K group in the matrix unit, then
// promotes that partial sum into a full FP32 accumulator, applying the
// group's dequantization scales at the same time.
//
// gfx950 mapping (not the pages' Hopper design, which overlapped two
// warpgroups so that one promotes while the other runs MMA):
//   * one v_mfma_scale_f32_16x16x128_f8f6f4 covers exactly one K group of a
//     16x16 output tile, so the partial sum P of a K group is a single
//     instruction issued with a zero accumulator (E8M0 operand scales = 1);
//   * promotion is acc = fma(P, sa(m,kb) * sb(kb,n), acc) on the VALU, which
//     the hardware overlaps with the next in-flight MFMAs of the same wave;
//   * workgroup tile 128x128, four waves in a 2x2 arrangement, each wave a
//     64x64 sub-tile = 4x4 MFMA tiles (64 FP32 accumulators per lane);
//   * A and B tiles (128 rows x 128 K bytes each) move HBM/L2 -> LDS with
//     global_load_lds_dwordx4 (no VGPR staging), double-buffered so the
//     next K group streams in while the current one is multiplied; rows are
//     stored with their 16-byte chunks XOR-swizzled by (row % 8) so that
//     the fragment reads of 8 consecutive rows hit distinct LDS banks;
//   * per-row scales of A (and per-column scales of B in the column mode)
//     ride along into LDS with global_load_lds_dword;
//   * workgroup ids are remapped so that consecutive tiles run on the same
//     XCD (each XCD has its own L2), and tiles are ordered in groups of 8
//     M-tiles so that co-resident workgroups share A and B panels.
// Grouped GEMM: the same tile kernel; a workgroup's linear tile id is
// resolved against the device-side expert offsets (expert-major order), so
// ragged and empty experts need no host synchronization.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace fp8fg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kE8M0One = 127;  // E8M0 encoding of 2^0

struct __align__(16) Stage {
  uint8_t a[kBM * kBK];
  uint8_t b[kBN * kBK];
  float sa[kBM];
  float sb[kBN];
};

struct KParams {
  int64_t M, N, K;
  const uint8_t* a;
  int64_t lda;
  const float* sa;
  int64_t sa_ms, sa_ks;
  const uint8_t* b;
  int64_t ldb;
  const float* sb;
  int64_t sb_ns, sb_ks;
  void* c;
  int64_t ldc;
  const int32_t* offsets;
  int64_t b_gs, sb_gs;
  int G;
  int tiles_n;
  int nblocks;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds, 4, 0, 0);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
// that each XCD receives a contiguous range of logical tile ids.
__device__ __forceinline__ int xcd_remap(int pid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int xcd = pid & 7, local = pid >> 3;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

// Logical id -> (tm, tn) in groups of kGroupM tile-rows.
__device__ __forceinline__ void grouped_order(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = id / per_group;
  const int first = g * kGroupM;
  const int gm = min(tiles_m - first, kGroupM);
  const int in = id - g * per_group;
  tm = first + in % gm;
  tn = in / gm;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int CT, int BMODE, bool NOPROMO, bool GROUPED>
__global__ __launch_bounds__(kThreads, 2) void gemm_blockscaled_kernel(KParams p) {
  __shared__ Stage stage[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // ---- tile decode
  const int id = xcd_remap(blockIdx.x, p.nblocks);
  const uint8_t* A = p.a;
  const uint8_t* B = p.b;
  const float* SB = p.sb;
  int64_t row_base;
  int rows_valid;
  int tn;
  if constexpr (GROUPED) {
    int t = id;
    int e = 0;
    int64_t seg0 = 0, seg1 = 0;
    bool found = false;
    for (; e < p.G; ++e) {
      seg0 = p.offsets[e];
      seg1 = p.offsets[e + 1];
      const int tm_e = (int)((seg1 - seg0 + kBM - 1) / kBM);
      const int cnt = tm_e * p.tiles_n;
      if (t < cnt) {
        int tm;
        grouped_order(t, tm_e, p.tiles_n, tm, tn);
        row_base = seg0 + (int64_t)tm * kBM;
        const int64_t rem = seg1 - row_base;
        rows_valid = rem < kBM ? (int)rem : kBM;
        found = true;
        break;
      }
      t -= cnt;
    }
    if (!found) return;
    B += (int64_t)e * p.b_gs;
    SB += (int64_t)e * p.sb_gs;
  } else {
    const int tiles_m = (int)((p.M + kBM - 1) / kBM);
    int tm;
    grouped_order(id, tiles_m, p.tiles_n, tm, tn);
    row_base = (int64_t)tm * kBM;
    const int64_t rem = p.M - row_base;
    rows_valid = rem < kBM ? (int)rem : kBM;
  }
  const int64_t n0 = (int64_t)tn * kBN;
  const int nkb = (int)(p.K / kBK);

  // ---- per-lane DMA sources.  Instruction i of wave w fills LDS rows
  // (4i + w) * 8 .. +8; lane l writes physical chunk l % 8 of row l / 8,
  // which holds logical K chunk (l % 8) ^ (row % 8).
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;
  const uint8_t* a_src[4];
  const uint8_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (i * 4 + wave) * 8 + lrow;
    const int ra = r < rows_valid ? r : rows_valid - 1;  // ragged M: repeat the last row
    a_src[i] = A + (row_base + ra) * p.lda + lchunk * 16;
    b_src[i] = B + (n0 + r) * p.ldb + lchunk * 16;
  }
  const float* sa_src[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = h * 64 + lane;
    const int ra = r < rows_valid ? r : rows_valid - 1;
    sa_src[h] = p.sa + (row_base + ra) * p.sa_ms;
  }
  const float* sbc_src[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) sbc_src[h] = SB + (n0 + h * 64 + lane) * p.sb_ns;

  auto issue = [&](int kb, Stage& S) {
    const int64_t koff = (int64_t)kb * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(a_src[i] + koff, S.a + (i * 4 + wave) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(b_src[i] + koff, S.b + (i * 4 + wave) * 1024);
    if (!NOPROMO && wave == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) dma4(sa_src[h] + kb * p.sa_ks, S.sa + h * 64);
    }
    if (!NOPROMO && BMODE == 1 && wave == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h) dma4(sbc_src[h] + kb * p.sb_ks, S.sb + h * 64);
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // B block scales: one value per K group for this tile's 128 columns (a
  // wave-uniform address, read through the scalar cache).
  const float* sb_blk = SB + __builtin_amdgcn_readfirstlane((int)(n0 >> 7)) * p.sb_ns;

  // sbv: block scale of B for the current K group, loaded one group ahead
  float sbv = 0.f;
  if (nkb > 0) {
    issue(0, stage[0]);
    if (!NOPROMO && BMODE == 0) sbv = sb_blk[0];
  }
  for (int kb = 0; kb < nkb; ++kb) {
    const Stage& S = stage[kb & 1];
    wait_vmcnt0();   // this wave's copies of K group kb have landed in LDS
    __syncthreads(); // ... and everyone's; stage (kb+1)&1 is free again

    // ---- fragments: lane l supplies row l % 16 and K bytes [32 (l/16), +32)
    v8i af[4], bf[4];
    const int fr = lane & 15;
    const int fc = (lane >> 4) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 64 + i * 16 + fr;
      const int sw = row & 7;
      const uint4 lo = *reinterpret_cast<const uint4*>(S.a + row * 128 + ((fc ^ sw) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(S.a + row * 128 + (((fc + 1) ^ sw) << 4));
      af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 64 + j * 16 + fr;
      const int sw = row & 7;
      const uint4 lo = *reinterpret_cast<const uint4*>(S.b + row * 128 + ((fc ^ sw) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(S.b + row * 128 + (((fc + 1) ^ sw) << 4));
      bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    // output rows of this lane within each 16x16 tile: 4 (l/16) + r
    float sar[4][4];
    float sbc[4];
    if constexpr (!NOPROMO) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 t = *reinterpret_cast<const float4*>(S.sa + wm * 64 + i * 16 + 4 * (lane >> 4));
        sar[i][0] = t.x; sar[i][1] = t.y; sar[i][2] = t.z; sar[i][3] = t.w;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sbc[j] = BMODE == 1 ? S.sb[wn * 64 + j * 16 + fr] : 1.0f;
    }

    // All reads of this stage are issued above, so the copies of the next
    // K group (into the other stage) can start now and overlap the MFMAs.
    float sbv_next = 0.f;
    if (kb + 1 < nkb) {
      issue(kb + 1, stage[(kb + 1) & 1]);
      if (!NOPROMO && BMODE == 0) sbv_next = sb_blk[(int64_t)(kb + 1) * p.sb_ks];
    }

    if constexpr (NOPROMO) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[i], bf[j], acc[i][j], 0, 0, 0, kE8M0One, 0, kE8M0One);
    } else {
      if constexpr (BMODE == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) sar[i][r] *= sbv;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sbj = sbc[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[i], bf[j], zero, 0, 0, 0, kE8M0One, 0, kE8M0One);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sc = BMODE == 0 ? sar[i][r] : sar[i][r] * sbj;
            acc[i][j][r] = __builtin_fmaf(P[r], sc, acc[i][j][r]);
          }
        }
      }
    }
    sbv = sbv_next;
  }

  // ---- epilogue: lane holds C[4 (l/16) + r][l % 16] of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * 64 + i * 16 + 4 * (lane >> 4) + r;
      if (row >= rows_valid) continue;
      const int64_t grow = row_base + row;
      float rs = 1.0f;
      if constexpr (NOPROMO) rs = p.sa[grow * p.sa_ms];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
        float v = acc[i][j][r];
        if constexpr (NOPROMO) {
          const float cs = BMODE == 0 ? sb_blk[0] : SB[col * p.sb_ns];
          v = v * (rs * cs);
        }
        if constexpr (CT == 0) {
          reinterpret_cast<uint16_t*>(p.c)[grow * p.ldc + col] = f32_to_bf16_rne(v);
        } else {
          reinterpret_cast<float*>(p.c)[grow * p.ldc + col] = v;
        }
      }
    }
  }
}

template <int CT, int BMODE, bool NOPROMO, bool GROUPED>
hipError_t launch_t(const KParams& kp, hipStream_t st) {
  hipLaunchKernelGGL((gemm_blockscaled_kernel<CT, BMODE, NOPROMO, GROUPED>), dim3(kp.nblocks),
                     dim3(kThreads), 0, st, kp);
  return hipGetLastError();
}

template <int CT, int BMODE>
hipError_t launch_mode(const KParams& kp, bool nopromo, bool grouped, hipStream_t st) {
  if (grouped) {
    return nopromo ? launch_t<CT, BMODE, true, true>(kp, st) : launch_t<CT, BMODE, false, true>(kp, st);
  }
  return nopromo ? launch_t<CT, BMODE, true, false>(kp, st) : launch_t<CT, BMODE, false, false>(kp, st);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  KParams kp;
  kp.M = g.M;
  kp.N = g.N;
  kp.K = g.K;
  kp.a = g.a;
  kp.lda = g.lda;
  kp.sa = g.sa;
  kp.sa_ms = g.sa_ms;
  kp.sa_ks = g.sa_ks;
  kp.b = g.b;
  kp.ldb = g.ldb;
  kp.sb = g.sb;
  kp.sb_ns = g.sb_ns;
  kp.sb_ks = g.sb_ks;
  kp.c = g.c;
  kp.ldc = g.ldc;
  kp.offsets = g.offsets;
  kp.b_gs = g.b_gs;
  kp.sb_gs = g.sb_gs;
  kp.G = (int)g.G;
  kp.tiles_n = (int)(g.N / kBN);
  const bool grouped = g.G > 0;
  const int64_t tiles_m = grouped ? (g.M + kBM - 1) / kBM + g.G : (g.M + kBM - 1) / kBM;
  const int64_t nblocks = tiles_m * kp.tiles_n;
  if (nblocks == 0) return hipSuccess;
  kp.nblocks = (int)nblocks;
  if (g.c_type == 0) {
    return g.b_scale_mode == 0 ? launch_mode<0, 0>(kp, g.no_promotion, grouped, st)
                               : launch_mode<0, 1>(kp, g.no_promotion, grouped, st);
  }
  return g.b_scale_mode == 0 ? launch_mode<1, 0>(kp, g.no_promotion, grouped, st)
                             : launch_mode<1, 1>(kp, g.no_promotion, grouped, st);
}

}  // namespace fp8fg
