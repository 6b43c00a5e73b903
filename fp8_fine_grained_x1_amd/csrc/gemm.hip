// Block-scaled FP8 GEMM (dense and grouped) for gfx950.
//
// The method ([thedaegu] Figure 7(b) passage; [fooled] promotion paragraph;
// [hearaon] accumulation-precision paragraph; page keys in
// include/fp8fg.h): an FP8 GEMM whose operands carry one scale per 128
// elements of K forms the partial sum of each 128-wide K group in the
// matrix unit, then promotes it into a full FP32 accumulator, applying the
// group's dequantization scales at the same time.
//
// gfx950 finding that shapes this kernel: the FP8 MFMA instructions
// (v_mfma_*_f8f6f4 and the older *_fp8_fp8) add the products of every 8
// consecutive K elements at a precision of about 14 bits below the largest
// of them (smaller products are cut off), before the 8-product sums are
// accumulated in FP32.  That is the same kind of limitation the pages
// measured on Hopper tensor cores, but it sits *inside* one instruction, so
// no promotion interval can remove it (relative Frobenius error ~5e-5 on
// the reference workloads).  The BF16 MFMA has no such loss.  Hence:
//
// default path (MODE 0, exact partial sums):
//   * the FP8 tiles stay FP8 in HBM and LDS (half the bytes of BF16);
//   * each wave converts its fragments FP8 -> BF16 in registers with
//     v_cvt_scalef32_pk_bf16_fp8 (scale 1.0: exact, every E4M3 value is a
//     BF16 value) and runs v_mfma_f32_32x32x16_bf16, chaining the 8
//     16-wide K steps of a K group in one accumulator P;
//   * promotion acc = fma(P, sa(m,kb) * sb(kb,n), acc) on the VALU, once per
//     output element and K group.
// FP8 paths (flags): MODE 1 forms P with one v_mfma_scale_f32_16x16x128_f8f6f4
//   per 16x16 tile and K group (E8M0 operand scales = 1), then promotes as
//   above; MODE 2 (no promotion) chains the FP8 MFMA over the whole K and
//   applies per-tensor scales once -- the naive baseline.
//
// Shared structure:
//   * workgroup tile 128x128, four waves in a 2x2 arrangement, each wave a
//     64x64 sub-tile;
//   * A and B tiles (128 rows x 128 K bytes each) move HBM/L2 -> LDS with
//     buffer_load_dwordx4 ... lds (no VGPR staging; the K offset rides in an
//     SGPR), double-buffered so the next K group streams in while the current
//     one is multiplied; the 16-byte chunks of each 128-byte row are
//     XOR-swizzled by (row / 2) % 8 so that fragment reads of 16 consecutive
//     rows hit distinct LDS banks;
//   * per-row scales of A (and per-column scales of B in the column mode) are
//     loaded into registers two K groups ahead and written into a separate
//     LDS object one group ahead, so that neither ever waits for the tile
//     copies in flight; a B block scale is one wave-uniform load per K group,
//     issued a group ahead;
//   * workgroup ids are remapped so that consecutive tiles run on the same
//     XCD (each XCD has its own L2), and tiles are ordered in groups of 8
//     M-tiles so that co-resident workgroups share A and B panels.
// Grouped GEMM: the same tile kernel; a workgroup's linear tile id is
// resolved against the device-side expert offsets (expert-major order), so
// ragged and empty experts need no host synchronization.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "fp8fg.h"
#include "launch.h"

namespace fp8fg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kE8M0One = 127;  // E8M0 encoding of 2^0

constexpr int kModeExact = 0;     // BF16 MFMA partial sums
constexpr int kModeFp8 = 1;       // FP8 MFMA partial sums, promoted
constexpr int kModeFp8NoPromo = 2;

struct __align__(16) Stage {
  uint8_t a[kBM * kBK];
  uint8_t b[kBN * kBK];
};
// Scales of one K group (A rows; B columns in the per-column mode).
struct __align__(16) Scales {
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

// Buffer resource over [base, base + bytes) (gfx9 raw buffer, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from rsrc + voffset + soffset into lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset,
                                      void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voffset, soffset, 0, 0);
}
// LDS tile layout: row r of a 128-byte-per-row tile keeps logical 16-byte
// chunk c at physical chunk c ^ swz(r).  With 64 LDS banks a 16-byte read by
// 16 consecutive lanes covers 16 consecutive rows; swz(r) = (r / 2) % 8 puts
// them in 16 distinct bank groups (rows r and r + 1 differ in the upper/lower
// half of the 256-byte bank window).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

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

template <int CT>
__device__ __forceinline__ void store_c(void* c, int64_t idx, float v) {
  if constexpr (CT == 0) {
    reinterpret_cast<uint16_t*>(c)[idx] = f32_to_bf16_rne(v);
  } else {
    reinterpret_cast<float*>(c)[idx] = v;
  }
}

// 8 E4M3 bytes (two dwords) -> 8 BF16 values, exactly.
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  union {
    v2bf p[4];
    v8bf v;
  } u;
  u.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
  u.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
  u.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
  u.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
  return u.v;
}

template <int CT, int BMODE, int MODE, bool GROUPED>
__global__ __launch_bounds__(kThreads, 2) void gemm_blockscaled_kernel(KParams p) {
  constexpr bool kPromote = MODE != kModeFp8NoPromo;
  // Two stages of tiles and two of scales, each its own LDS object: with the
  // K loop unrolled by two every access names its object at compile time, so
  // the compiler can tell copies in flight into one stage from reads of the
  // other and inserts no wait between them.
  __shared__ Stage stage0;
  __shared__ Stage stage1;
  __shared__ Scales scales0;
  __shared__ Scales scales1;

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
  int64_t row_base = 0;
  int rows_valid = 0;
  int tn = 0;
  if constexpr (GROUPED) {
    int t = id;
    int e = 0;
    bool found = false;
    for (; e < p.G; ++e) {
      const int64_t seg0 = p.offsets[e];
      const int64_t seg1 = p.offsets[e + 1];
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

  // ---- per-lane copy sources.  Instruction i of wave w fills LDS rows
  // (4i + w) * 8 .. +8; lane l writes physical chunk l % 8 of row l / 8,
  // which holds logical K chunk (l % 8) ^ swz(row).  Tile-relative byte
  // offsets go in the VGPR offset, the K group's offset in the SGPR offset.
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + row_base * p.lda, (uint32_t)(rows_valid * p.lda));
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + n0 * p.ldb, (uint32_t)(kBN * p.ldb));
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (i * 4 + wave) * 8 + (lane >> 3);
    const int ra = r < rows_valid ? r : rows_valid - 1;  // ragged M: repeat the last row
    const int lchunk = (lane & 7) ^ swz(r);
    a_off[i] = (uint32_t)(ra * p.lda + lchunk * 16);
    b_off[i] = (uint32_t)(r * p.ldb + lchunk * 16);
  }
  // scales: lane l of wave 0 (A rows) / wave 1 (B columns in the per-column
  // mode) copies entries l and l + 64 of the K group
  const bool scale_wave = kPromote && (wave == 0 || (BMODE == 1 && wave == 1));
  const float* sc_src0;
  const float* sc_src1;
  int64_t sc_ks;
  if (wave == 0) {
    const int r0 = lane < rows_valid ? lane : rows_valid - 1;
    const int r1 = lane + 64 < rows_valid ? lane + 64 : rows_valid - 1;
    sc_src0 = p.sa + (row_base + r0) * p.sa_ms;
    sc_src1 = p.sa + (row_base + r1) * p.sa_ms;
    sc_ks = p.sa_ks;
  } else {
    sc_src0 = SB + (n0 + lane) * p.sb_ns;
    sc_src1 = SB + (n0 + lane + 64) * p.sb_ns;
    sc_ks = p.sb_ks;
  }

  // Copies of K group kb's tiles into stage S (LDS DMA, no VGPRs).
  auto issue = [&](int kb, Stage& S) {
    const uint32_t koff = (uint32_t)kb * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(a_rsrc, a_off[i], koff, S.a + (i * 4 + wave) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(b_rsrc, b_off[i], koff, S.b + (i * 4 + wave) * 1024);
  };
  // Scales travel global -> VGPR -> LDS: loaded two K groups ahead (so the
  // wait at the top of the next group already covers them) and written into
  // their own LDS object at the end of the group before their use.
  // B block scales: one value per K group for this tile's 128 columns.
  const float* sb_blk = SB + __builtin_amdgcn_readfirstlane((int)(n0 >> 7)) * p.sb_ns;
  // In the block mode the B scale of the K group is folded in before the
  // store (LDS then holds sa(m, kb) * sb(kb, n0 / 128)), so the promotion is
  // a single FMA per element.
  auto load_scales = [&](int kb, float (&v)[3]) {
    if (scale_wave) {
      v[0] = sc_src0[(int64_t)kb * sc_ks];
      v[1] = sc_src1[(int64_t)kb * sc_ks];
      if (BMODE == 0) v[2] = sb_blk[(int64_t)kb * p.sb_ks];
    }
  };
  auto store_scales = [&](Scales& SC, const float (&v)[3]) {
    if (scale_wave) {
      float* dst = wave == 0 ? SC.sa : SC.sb;
      const float f = (BMODE == 0 && wave == 0) ? v[2] : 1.0f;
      dst[lane] = v[0] * f;
      dst[lane + 64] = v[1] * f;
    }
  };
  float scr0[3] = {0.f, 0.f, 0.f}, scr1[3] = {0.f, 0.f, 0.f};  // scale registers, two sets


  if constexpr (MODE == kModeExact) {
    // ================================================================ BF16 MFMA
    // Wave tile 64x64 = 2x2 tiles of 32x32.  Lane l serves row/column l % 32
    // of a tile; lane group g = l / 32 takes K bytes [64 g, 64 g + 64) of each
    // K group, 8 per 16-wide K step (the same permutation of K for A and B).
    // Accumulator layout of v_mfma_f32_32x32x16_bf16: element r of lane l is
    // row 8 (r / 4) + 4 g + r % 4, column l % 32.
    const int g = lane >> 5;
    const int lr = lane & 31;
    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Pipeline inside a K group: the 16-byte chunk holding K steps 2c, 2c+1
    // is read from LDS about two steps before its first use, and the BF16
    // fragments of step s + 1 are converted while the 4 MFMAs of step s run
    // (interleaved one MFMA : four conversions).
    auto group = [&](int kb, const Stage& S, const Scales& SS, Stage& Nx,
                     float (&sc_store)[3], float (&sc_load)[3], Scales& NS) {
      wait_vmcnt0();    // this wave's copies of K group kb have landed in LDS
      __syncthreads();  // ... and everyone's; the other stage is free again
      uint4 ra[4][2], rb[4][2];
      auto read_chunk = [&](int c) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = wm * 64 + i * 32 + lr;
          ra[c][i] = *reinterpret_cast<const uint4*>(S.a + row * 128 + (((4 * g + c) ^ swz(row)) << 4));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = wn * 64 + j * 32 + lr;
          rb[c][j] = *reinterpret_cast<const uint4*>(S.b + row * 128 + (((4 * g + c) ^ swz(row)) << 4));
        }
      };
      v8bf af[2][2], bf[2][2];  // [step parity][tile]
      auto convert = [&](int st) {
        const int c = st >> 1, h = st & 1, par = st & 1;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[par][i] = h ? fp8x8_to_bf16(ra[c][i].z, ra[c][i].w) : fp8x8_to_bf16(ra[c][i].x, ra[c][i].y);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bf[par][j] = h ? fp8x8_to_bf16(rb[c][j].z, rb[c][j].w) : fp8x8_to_bf16(rb[c][j].x, rb[c][j].y);
      };
      read_chunk(0);
      read_chunk(1);
      __builtin_amdgcn_sched_barrier(0);
      // copies of the next K group, issued after this group's first reads
      if (kb + 1 < nkb) issue(kb + 1, Nx);
      if (kb + 2 < nkb) load_scales(kb + 2, sc_load);
      convert(0);
      __builtin_amdgcn_sched_barrier(0);
      v16f P[2][2];
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int par = st & 1;
        if ((st & 1) && (st >> 1) + 2 < 4) read_chunk((st >> 1) + 2);
        if (st + 1 < 8) convert(st + 1);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (st == 0) {
              const v16f z = {};
              P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[par][i], bf[par][j], z, 0, 0, 0);
            } else {
              P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[par][i], bf[par][j], P[i][j], 0, 0, 0);
            }
          }
        if ((st & 1) && (st >> 1) + 2 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (st + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // promotion: the scales of this lane's rows are tile i, rows 8 q + 4 g + t
      float sbc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) sbc[j] = BMODE == 1 ? SS.sb[wn * 64 + j * 32 + lr] : 1.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 s4 = *reinterpret_cast<const float4*>(SS.sa + wm * 64 + i * 32 + 8 * q + 4 * g);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float sc = BMODE == 1 ? sv[t] * sbc[j] : sv[t];
              acc[i][j][4 * q + t] = __builtin_fmaf(P[i][j][4 * q + t], sc, acc[i][j][4 * q + t]);
            }
          }
        }
      if (kb + 1 < nkb) store_scales(NS, sc_store);
    };

    if (nkb > 0) {
      load_scales(0, scr0);
      if (nkb > 1) load_scales(1, scr1);
      store_scales(scales0, scr0);
      issue(0, stage0);
    }
    for (int kb = 0; kb < nkb; kb += 2) {
      group(kb, stage0, scales0, stage1, scr1, scr0, scales1);
      if (kb + 1 < nkb) group(kb + 1, stage1, scales1, stage0, scr0, scr1, scales0);
    }

    // ---- epilogue
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row >= rows_valid) continue;
        const int64_t grow = row_base + row;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = n0 + wn * 64 + j * 32 + lr;
          store_c<CT>(p.c, grow * p.ldc + col, acc[i][j][r]);
        }
      }
  } else {
    // ================================================================ FP8 MFMA
    // Wave tile 64x64 = 4x4 tiles of 16x16.  Lane l supplies row l % 16 and K
    // bytes [32 (l/16), +32) of a K group; accumulator element r of lane l is
    // row 4 (l/16) + r, column l % 16.
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int fr = lane & 15;
    const int fc = (lane >> 4) * 2;

    auto group = [&](int kb, const Stage& S, const Scales& SS, Stage& Nx,
                     float (&sc_store)[3], float (&sc_load)[3], Scales& NS) {
      wait_vmcnt0();
      __syncthreads();
      if (kb + 1 < nkb) issue(kb + 1, Nx);
      if (kb + 2 < nkb) load_scales(kb + 2, sc_load);
      v8i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + fr;
        const int sw = swz(row);
        const uint4 lo = *reinterpret_cast<const uint4*>(S.a + row * 128 + ((fc ^ sw) << 4));
        const uint4 hi = *reinterpret_cast<const uint4*>(S.a + row * 128 + (((fc + 1) ^ sw) << 4));
        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wn * 64 + j * 16 + fr;
        const int sw = swz(row);
        const uint4 lo = *reinterpret_cast<const uint4*>(S.b + row * 128 + ((fc ^ sw) << 4));
        const uint4 hi = *reinterpret_cast<const uint4*>(S.b + row * 128 + (((fc + 1) ^ sw) << 4));
        bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      if constexpr (!kPromote) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af[i], bf[j], acc[i][j], 0, 0, 0, kE8M0One, 0, kE8M0One);
      } else {
        float sar[4][4];
        float sbc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 t = *reinterpret_cast<const float4*>(SS.sa + wm * 64 + i * 16 + 4 * (lane >> 4));
          sar[i][0] = t.x; sar[i][1] = t.y; sar[i][2] = t.z; sar[i][3] = t.w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sbc[j] = BMODE == 1 ? SS.sb[wn * 64 + j * 16 + fr] : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af[i], bf[j], zero, 0, 0, 0, kE8M0One, 0, kE8M0One);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i][j][r] = __builtin_fmaf(P[r], sar[i][r] * sbc[j], acc[i][j][r]);
          }
        }
      }
      if (kb + 1 < nkb) store_scales(NS, sc_store);
    };

    if (nkb > 0) {
      load_scales(0, scr0);
      if (nkb > 1) load_scales(1, scr1);
      store_scales(scales0, scr0);
      issue(0, stage0);
    }
    for (int kb = 0; kb < nkb; kb += 2) {
      group(kb, stage0, scales0, stage1, scr1, scr0, scales1);
      if (kb + 1 < nkb) group(kb + 1, stage1, scales1, stage0, scr0, scr1, scales0);
    }

    // ---- epilogue
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (row >= rows_valid) continue;
        const int64_t grow = row_base + row;
        float rs = 1.0f;
        if constexpr (!kPromote) rs = p.sa[grow * p.sa_ms];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
          float v = acc[i][j][r];
          if constexpr (!kPromote) {
            const float cs = BMODE == 0 ? sb_blk[0] : SB[col * p.sb_ns];
            v = v * (rs * cs);
          }
          store_c<CT>(p.c, grow * p.ldc + col, v);
        }
      }
    }
  }
}

template <int CT, int BMODE, int MODE, bool GROUPED>
hipError_t launch_t(const KParams& kp, hipStream_t st) {
  hipLaunchKernelGGL((gemm_blockscaled_kernel<CT, BMODE, MODE, GROUPED>), dim3(kp.nblocks),
                     dim3(kThreads), 0, st, kp);
  return hipGetLastError();
}

template <int CT, int BMODE, int MODE>
hipError_t launch_grouped_or_dense(const KParams& kp, bool grouped, hipStream_t st) {
  return grouped ? launch_t<CT, BMODE, MODE, true>(kp, st) : launch_t<CT, BMODE, MODE, false>(kp, st);
}

template <int CT, int BMODE>
hipError_t launch_mode(const KParams& kp, int mode, bool grouped, hipStream_t st) {
  switch (mode) {
    case kModeExact: return launch_grouped_or_dense<CT, BMODE, kModeExact>(kp, grouped, st);
    case kModeFp8: return launch_grouped_or_dense<CT, BMODE, kModeFp8>(kp, grouped, st);
    default: return launch_grouped_or_dense<CT, BMODE, kModeFp8NoPromo>(kp, grouped, st);
  }
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
  const int mode = (g.flags & FP8FG_GEMM_NO_PROMOTION) ? kModeFp8NoPromo
                   : (g.flags & FP8FG_GEMM_FP8_MFMA)   ? kModeFp8
                                                        : kModeExact;
  if (g.c_type == 0) {
    return g.b_scale_mode == 0 ? launch_mode<0, 0>(kp, mode, grouped, st)
                               : launch_mode<0, 1>(kp, mode, grouped, st);
  }
  return g.b_scale_mode == 0 ? launch_mode<1, 0>(kp, mode, grouped, st)
                             : launch_mode<1, 1>(kp, mode, grouped, st);
}

}  // namespace fp8fg
