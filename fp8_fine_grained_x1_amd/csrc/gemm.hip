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
// Kernels (which one runs is decided on the host from the arguments):
//   * gemm_rescale_kernel -- the default path with 128x128 B block scales:
//     exact partial sums (the FP8 fragments are converted to BF16 in
//     registers with v_cvt_scalef32_pk_bf16_fp8, scale 1.0, which is exact,
//     and multiplied with v_mfma_f32_32x32x16_bf16) accumulated in units of
//     the current K group's scale, the accumulator rescaled once per group;
//     256 x 256 and 256 x 192 tiles (described before the kernel);
//   * gemm_rescale_grouped_kernel -- the same for grouped launches, where
//     an expert's last tile of at most 128 rows runs as a 128-row tile;
//   * gemm_stream_kernel -- the same arithmetic for few rows per expert
//     (MoE decode) or a dense M <= 64: 64 x 128 tiles, weight streaming;
//   * gemm_mx_kernel -- the E8M0-scale flag with block scales and N a
//     multiple of 256: 256 x 256 tiles of v_mfma_scale_f32_32x32x64_f8f6f4,
//     the FP8 operands unconverted, the scales' powers of two as the
//     instruction's operand scales, the accumulator chained through the
//     instruction and kept in units of the leftover factors (described
//     before the kernel);
//   * gemm_blockscaled_kernel -- promotion of separate K-group partial sums:
//     MODE 0 (exact, as above) for per-column B scales and N = 128; the FP8
//     paths behind flags: MODE 1 forms P with one
//     v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 tile and K group (E8M0
//     operand scales = 1) and promotes acc = fma(P, sa * sb, acc); MODE 2
//     (no promotion) chains the FP8 MFMA over the whole K and applies
//     per-tensor scales once -- the naive baseline; MODE 3 gives each group's
//     scales to the instruction as its E8M0 operand scales (their powers of
//     two), so the products are dequantized inside the matrix unit and only
//     a remaining factor, 1 for power-of-two scales, meets the FP32
//     accumulate.
//
// gemm_blockscaled_kernel structure:
//   * workgroup tile 256 (M) x 128 (N), eight waves in a 4x2 arrangement,
//     each wave a 64x64 sub-tile; one workgroup per CU;
//   * A and B tiles (256 + 128 rows x 128 K bytes = 48 KB per K group) move
//     HBM/L2 -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging; the K
//     offset rides in an SGPR) through three LDS stages, so the copies of
//     K group kb + 2 stream in while kb is multiplied; the wait at the top of
//     a group leaves the newest group's copies in flight (vmcnt = copies per
//     group); the 16-byte chunks of each 128-byte row are XOR-swizzled by
//     (row / 2) % 8 so that fragment reads of 16 consecutive rows hit
//     distinct LDS banks;
//   * the MFMA operands are passed B-first, so the accumulator of a lane
//     holds one output row (and 4-element runs of columns): the row scale of
//     A is then one value per lane and MFMA tile, loaded straight from
//     global memory into registers two K groups ahead; a B block scale is one
//     value per K group (all lanes load it); per-column B scales go through a
//     small per-wave LDS array;
//   * workgroup ids are remapped so that consecutive tiles run on the same
//     XCD (each XCD has its own L2), and tiles are ordered in groups of
//     M-tiles so that co-resident workgroups share A and B panels.
// Grouped GEMM: the same kernels; a workgroup's linear tile id is resolved
// against the device-side expert offsets (expert-major order), so ragged and
// empty experts need no host synchronization.
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

constexpr int kBM = 256;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupM = 4;
constexpr int kE8M0One = 127;  // E8M0 encoding of 2^0
// One buffer_load ... lds of a wave moves 64 lanes x 16 B = 8 rows of 128 B.
constexpr int kDmaA = kBM / (8 * kWaves);  // per thread and K group
constexpr int kDmaB = kBN / (8 * kWaves);
constexpr int kDmaPerGroup = kDmaA + kDmaB;

constexpr int kModeExact = 0;     // BF16 MFMA partial sums
constexpr int kModeFp8 = 1;       // FP8 MFMA partial sums, promoted
constexpr int kModeFp8NoPromo = 2;
constexpr int kModeFp8Mx = 3;     // FP8 MFMA applying the scales' powers of two as E8M0 operand scales

struct __align__(16) Stage {
  uint8_t a[kBM * kBK];
  uint8_t b[kBN * kBK];
  // per-column B scales of the stage's K group, one copy per wave (columns
  // wn*64 .. +64); filled by the same LDS copies as the tiles, so that reads
  // of it wait only for this stage's copies
  float colsc[kWaves][64];
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
  int vec_store;   // c rows allow 4-element vector stores
  int64_t n_base;  // first output column of this launch's tiles
};

// Compile-time flags for generic lambdas.
template <int V>
struct IntTag {
  static constexpr int value = V;
};
template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over [base, base + bytes) (gfx9 raw buffer, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from rsrc + voffset + soffset into lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset,
                                      void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voffset, soffset, 0, 0);
}
// 4 bytes per lane into lds + 4 * lane.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset,
                                     void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voffset, soffset, 0, 0);
}
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voffset, (int)soffset, 0));
}
// LDS tile layout: row r of a 128-byte-per-row tile keeps logical 16-byte
// chunk c at physical chunk c ^ swz(r).  With 64 LDS banks a 16-byte read by
// 16 consecutive lanes covers 16 consecutive rows; swz(r) = (r / 2) % 8 puts
// them in 16 distinct bank groups (rows r and r + 1 differ in the upper/lower
// half of the 256-byte bank window).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima; gfx9 splits
// vmcnt over bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// s_waitcnt vmcnt(0) lgkmcnt(0): this wave's copies have landed and its LDS
// reads have returned their data.
__device__ __forceinline__ void wait_copies_and_reads() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Workgroup barrier without a memory fence: __syncthreads() would also wait
// for every copy in flight (vmcnt(0)).  Each wave has already waited for
// the copies the next group reads (explicit vmcnt above), and LDS reads of
// the stage about to be refilled completed before their MFMAs; the empty
// asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
// that each XCD receives a contiguous range of logical tile ids.
__device__ __forceinline__ int xcd_remap(int pid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int xcd = pid & 7, local = pid >> 3;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

// Logical tile id of this workgroup, or -1 if it has none.  A grouped
// launch is sized for the worst case (the sum of ceil(M_e / bm) is at most
// ceil(M / bm) + G row tiles): the tiles that exist are counted from the
// offsets, workgroups past that count have no tile, and the others are
// renumbered over the count, so that every XCD gets an equal contiguous
// share of real tiles rather than the empty ones piling up on the last XCDs.
template <bool GROUPED>
__device__ __forceinline__ int tile_id(const KParams& p, int bm) {
  if constexpr (!GROUPED) {
    return xcd_remap(blockIdx.x, p.nblocks);
  } else {
    int total = 0;
    for (int e = 0; e < p.G; ++e) {
      const int64_t rows = (int64_t)p.offsets[e + 1] - p.offsets[e];
      total += (int)((rows + bm - 1) / bm) * p.tiles_n;
    }
    if ((int)blockIdx.x >= total) return -1;
    return xcd_remap(blockIdx.x, total);
  }
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

// True when the FP32 product s = a * b of two nonzero scales lies below the
// normal range (it then carries fewer than 24 significant bits).
__device__ __forceinline__ bool scale_product_inexact(float a, float b, float s) {
  return __builtin_fabsf(s) < 1.17549435e-38f && a != 0.f && b != 0.f;
}

// Round to nearest even (hardware conversion; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

template <int CT>
__device__ __forceinline__ void store_c(void* c, int64_t idx, float v) {
  if constexpr (CT == 0) {
    reinterpret_cast<uint16_t*>(c)[idx] = f32_to_bf16(v);
  } else {
    reinterpret_cast<float*>(c)[idx] = v;
  }
}
// Four consecutive outputs c[idx .. idx + 3]; one 8-byte (bf16) or 16-byte
// (f32) store when the row layout allows it.
template <int CT>
__device__ __forceinline__ void store_c4(void* c, int64_t idx, const float (&v)[4], bool vec) {
  if (vec) {
    if constexpr (CT == 0) {
      uint2 u;
      u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(c) + idx) = u;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + idx) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) store_c<CT>(c, idx + t, v[t]);
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
__global__ __launch_bounds__(kThreads, 1) void gemm_blockscaled_kernel(KParams p) {
  constexpr bool kPromote = MODE != kModeFp8NoPromo;
  constexpr int kT = MODE == kModeExact ? 32 : 16;  // MFMA tile edge
  constexpr int kTiles = 64 / kT;                   // MFMA tiles per wave along M (and N)
  // Three stages of tiles, each its own LDS object: with the K loop unrolled
  // by three every access names its object at compile time, so the compiler
  // can tell copies in flight into one stage from reads of another and
  // inserts no wait between them.
  __shared__ Stage stage0;
  __shared__ Stage stage1;
  __shared__ Stage stage2;
  constexpr bool kColDma = kPromote && BMODE == 1;  // column scales travel with the tiles
  constexpr int kVmemWait = kDmaPerGroup + (kColDma ? 1 : 0);
  static_assert(kDmaPerGroup <= 8, "one tile copy per K step");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // ---- tile decode
  const int id = tile_id<GROUPED>(p, kBM);
  if (id < 0) return;
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
  // (8i + w) * 8 .. +8; lane l writes physical chunk l % 8 of row l / 8,
  // which holds logical K chunk (l % 8) ^ swz(row).  Tile-relative byte
  // offsets go in the VGPR offset, the K group's offset in the SGPR offset.
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + row_base * p.lda, (uint32_t)(rows_valid * p.lda));
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + n0 * p.ldb, (uint32_t)(kBN * p.ldb));
  uint32_t a_off[kDmaA], b_off[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    const int ra = r < rows_valid ? r : rows_valid - 1;  // ragged M: repeat the last row
    a_off[i] = (uint32_t)(ra * p.lda + (((lane & 7) ^ swz(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    b_off[i] = (uint32_t)(r * p.ldb + (((lane & 7) ^ swz(r)) << 4));
  }
  // ---- scale sources (buffer loads: 32-bit offsets, checked on the host).
  // A: this lane's output row in MFMA tile i is wm*64 + i*kT + lane % kT.
  const __amdgpu_buffer_rsrc_t sa_rsrc = make_rsrc(p.sa + row_base * p.sa_ms, 0xFFFFFFFFu);
  uint32_t sa_off[kTiles];
#pragma unroll
  for (int i = 0; i < kTiles; ++i) {
    const int r = wm * 64 + i * kT + (lane & (kT - 1));
    sa_off[i] = (uint32_t)((r < rows_valid ? r : rows_valid - 1) * p.sa_ms * 4);
  }
  // B: block mode, the scale of this tile's 128 columns (same for all
  // lanes, into a register); per-column mode, column wn*64 + lane (copied
  // into the stage's per-wave column-scale array).
  const __amdgpu_buffer_rsrc_t sb_rsrc =
      make_rsrc(SB + (BMODE == 0 ? (n0 >> 7) : n0) * p.sb_ns, 0xFFFFFFFFu);
  const uint32_t sb_off = BMODE == 0 ? 0u : (uint32_t)((wn * 64 + lane) * p.sb_ns * 4);


  // A resource of size 0: loads through it fetch nothing and return zeros.
  const __amdgpu_buffer_rsrc_t null_rsrc = make_rsrc(p.a, 0u);
  // Copies of K group kb's tiles (and per-column B scales) into stage S (LDS
  // DMA, no VGPRs).  Every group issues the same number of copies, so that
  // the wait counts hold on every path; past the last K group they go
  // through the empty resource (zeros into a stage that is not read again).
  // Copy number `idx` (0 .. kVmemWait - 1) of K group kb; the copies of one
  // group are spread over its K steps so that the address queues never fill
  // and no wave stalls at issue.
  auto issue_one = [&](int kb, Stage& S, int idx) {
    const bool live = kb < nkb;
    const uint32_t koff = live ? (uint32_t)kb * kBK : 0u;
    if (idx < kDmaA) {
      dma16(live ? a_rsrc : null_rsrc, a_off[idx], koff, S.a + (idx * kWaves + wave) * 1024);
    } else if (idx < kDmaPerGroup) {
      const int i = idx - kDmaA;
      dma16(live ? b_rsrc : null_rsrc, b_off[i], koff, S.b + (i * kWaves + wave) * 1024);
    } else if constexpr (kColDma) {
      dma4(live ? sb_rsrc : null_rsrc, sb_off, live ? (uint32_t)(kb * p.sb_ks * 4) : 0u, &S.colsc[wave][0]);
    }
  };
  auto issue = [&](int kb, Stage& S) {
#pragma unroll
    for (int i = 0; i < kVmemWait; ++i) issue_one(kb, S, i);
  };
  // Row scales of A (and the B block scale) of group kb into registers.
  struct ScaleRegs {
    float sa[kTiles];
    float sb;
  };
  auto load_scales = [&](int kb, ScaleRegs& s) {
    if constexpr (kPromote) {
      const bool live = kb < nkb;
      const __amdgpu_buffer_rsrc_t ra = live ? sa_rsrc : null_rsrc;
      const uint32_t ka = live ? (uint32_t)(kb * p.sa_ks * 4) : 0u;
#pragma unroll
      for (int i = 0; i < kTiles; ++i) s.sa[i] = load_f32(ra, sa_off[i], ka);
      if constexpr (BMODE == 0)
        s.sb = load_f32(live ? sb_rsrc : null_rsrc, 0u, live ? (uint32_t)(kb * p.sb_ks * 4) : 0u);
    }
  };
  // Top of K group kb: its copies (and every older memory load) have
  // landed, for this wave and -- after the barrier -- for all; the stage
  // read in group kb - 1 is free again.  Only the copies of group kb + 1
  // (real or empty) may still be in flight.
  auto wait_group = [&]() {
    wait_vmcnt<kVmemWait>();
    block_barrier();
  };

  ScaleRegs sr0{}, sr1{}, sr2{};
  load_scales(0, sr0);
  issue(0, stage0);
  load_scales(1, sr1);
  issue(1, stage1);
  // The K loop: full triples of groups, then the remaining one or two.  No
  // group is conditional inside the loop, so on every control-flow path the
  // copies into the stage a group reads are followed by exactly one group's
  // copies, and the compiler's own wait analysis agrees with wait_group.
  auto k_loop = [&](auto& group) {
    int kb = 0;
    for (; kb + 3 <= nkb; kb += 3) {
      group(kb, stage0, sr0, stage2, sr2);
      group(kb + 1, stage1, sr1, stage0, sr0);
      group(kb + 2, stage2, sr2, stage1, sr1);
    }
    const int rem = nkb - kb;
    if (rem >= 1) {
      group(kb, stage0, sr0, stage2, sr2);
      if (rem == 2) group(kb + 1, stage1, sr1, stage0, sr0);
    }
  };

  if constexpr (MODE == kModeExact) {
    // ================================================================ BF16 MFMA
    // Wave tile 64x64 = 2x2 tiles of 32x32.  Lane l reads row l % 32 of an A
    // tile and of a B tile; lane group g = l / 32 takes K bytes
    // [64 g, 64 g + 64) of each K group, 8 per 16-wide K step (the same
    // permutation of K for A and B).  With B as the first MFMA operand the
    // accumulator element r of lane l is output row l % 32 and column
    // 8 (r / 4) + 4 g + r % 4 of the tile.
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
    auto group = [&](int kb, const Stage& S, const ScaleRegs& sr, Stage& Nx, ScaleRegs& nsr) {
      wait_group();
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
      // scales of K group kb + 2, after this group's first reads; its tile
      // copies follow one per K step below
      load_scales(kb + 2, nsr);
      if constexpr (kColDma) issue_one(kb + 2, Nx, kDmaPerGroup);
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
              P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[par][j], af[par][i], z, 0, 0, 0);
            } else {
              P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[par][j], af[par][i], P[i][j], 0, 0, 0);
            }
          }
        if (st < kDmaPerGroup) issue_one(kb + 2, Nx, st);
        if ((st & 1) && (st >> 1) + 2 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (st + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          if (m == 0 && st < kDmaPerGroup) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // promotion: tile i's row scale is one value per lane.  A scale
      // product below the FP32 normal range would lose precision, so a wave
      // with such a lane applies the two factors one after the other.
      if constexpr (BMODE == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float s = sr.sa[i] * sr.sb;
          if (__builtin_amdgcn_ballot_w64(scale_product_inexact(sr.sa[i], sr.sb, s)) == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(P[i][j][r], s, acc[i][j][r]);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(P[i][j][r] * sr.sa[i], sr.sb, acc[i][j][r]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 c4 = *reinterpret_cast<const float4*>(&S.colsc[wave][j * 32 + 8 * q + 4 * g]);
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int t = 0; t < 4; ++t)
                acc[i][j][4 * q + t] = __builtin_fmaf(P[i][j][4 * q + t] * sr.sa[i], cv[t], acc[i][j][4 * q + t]);
          }
      }
    };

    k_loop(group);
    wait_vmcnt<0>();  // no LDS copy may land after the workgroup ends

    // ---- epilogue: lane holds row lr of tile i, columns 8q + 4g .. +3 of tile j
    if constexpr (CT == 0) {
      const bool vec = p.vec_store != 0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + lr;
        if (row >= rows_valid) continue;
        const int64_t grow = row_base + row;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t col = n0 + wn * 64 + j * 32 + 8 * q + 4 * g;
            const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            store_c4<CT>(p.c, grow * p.ldc + col, v, vec);
          }
      }
    } else {
      // FP32 output: one copy of the stores per width, so that the aligned
      // copy keeps its 16-byte stores (with a per-store choice the compiler
      // merges the two forms into narrower ones).
      auto epilogue = [&](auto vec_c) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = wm * 64 + i * 32 + lr;
          if (row >= rows_valid) continue;
          const int64_t grow = row_base + row;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t col = n0 + wn * 64 + j * 32 + 8 * q + 4 * g;
              const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              store_c4<CT>(p.c, grow * p.ldc + col, v, decltype(vec_c)::value);
            }
        }
      };
      if (p.vec_store != 0)
        epilogue(BoolTag<true>{});
      else
        epilogue(BoolTag<false>{});
    }
  } else {
    // ================================================================ FP8 MFMA
    // Wave tile 64x64 = 4x4 tiles of 16x16.  Lane l supplies row l % 16 and K
    // bytes [32 (l/16), +32) of a K group; with B as the first operand the
    // accumulator element r of lane l is output row l % 16, column
    // 4 (l/16) + r of the tile.
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int fr = lane & 15;
    const int fc = (lane >> 4) * 2;

    auto group = [&](int kb, const Stage& S, const ScaleRegs& sr, Stage& Nx, ScaleRegs& nsr) {
      wait_group();
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
      float cv[4][4];
      float sbc[4];  // MODE 3, column scales: the column this lane supplies
      if constexpr (kColDma && MODE == kModeFp8Mx) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sbc[j] = S.colsc[wave][j * 16 + fr];
      } else if constexpr (kColDma) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 t = *reinterpret_cast<const float4*>(&S.colsc[wave][j * 16 + 4 * (lane >> 4)]);
          cv[j][0] = t.x; cv[j][1] = t.y; cv[j][2] = t.z; cv[j][3] = t.w;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // scales and copies of K group kb + 2, issued after this group's reads
      // (tile copies spread over the MFMAs, one every other one)
      load_scales(kb + 2, nsr);
      if constexpr (kColDma) issue_one(kb + 2, Nx, kDmaPerGroup);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!kPromote) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if ((j * 4 + i) % 2 == 0 && (j * 4 + i) / 2 < kDmaPerGroup) issue_one(kb + 2, Nx, (j * 4 + i) / 2);
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bf[j], af[i], acc[i][j], 0, 0, 0, kE8M0One, 0, kE8M0One);
          }
      } else if constexpr (MODE == kModeFp8Mx) {
        // Each scale s splits into its power of two 2^(E - 127) -- E its
        // exponent field, given to the instruction as an E8M0 operand scale
        // -- and the rest f = s * 2^(127 - E), exactly 1 for a power of two
        // (in [1, 2) otherwise, [0, 1) for 0 and denormals).  The lane that
        // supplies B column wn*64 + 16 j + l % 16 (the instruction's first
        // operand) gives that column's scale; the lane that supplies A row
        // wm*64 + 16 i + l % 16 gives that row's.  The group's partial sum
        // leaves the instruction scaled by the powers of two and is added to
        // acc times fa * fb: for power-of-two scales a plain FP32 add.
        int ea[4], eb[4];
        float fa[4], fb[4];
        auto split_scale = [](float sc, int& e, float& f) {
          e = (int)((__float_as_uint(sc) >> 23) & 0xFFu);
          f = __builtin_amdgcn_ldexpf(sc, 127 - e);
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) split_scale(sr.sa[i], ea[i], fa[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float sbj = sr.sb;
          if constexpr (BMODE == 1) sbj = sbc[j];
          split_scale(sbj, eb[j], fb[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if ((j * 4 + i) % 2 == 0 && (j * 4 + i) / 2 < kDmaPerGroup) issue_one(kb + 2, Nx, (j * 4 + i) / 2);
            const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], zero, 0, 0, 0, eb[j], 0, ea[i]);
            const float f = fa[i] * fb[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(P[r], f, acc[i][j][r]);
          }
      } else {
        if constexpr (!kColDma) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) cv[j][r] = sr.sb;
        }
        // block scales: one product per row tile unless some lane's product
        // lies below the FP32 normal range; column scales: the two factors
        // one after the other
        bool split = BMODE == 1;
        float s[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BMODE == 0) {
          bool bad = false;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[i] = sr.sa[i] * sr.sb;
            bad = bad || scale_product_inexact(sr.sa[i], sr.sb, s[i]);
          }
          split = __builtin_amdgcn_ballot_w64(bad) != 0;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if ((j * 4 + i) % 2 == 0 && (j * 4 + i) / 2 < kDmaPerGroup) issue_one(kb + 2, Nx, (j * 4 + i) / 2);
            const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bf[j], af[i], zero, 0, 0, 0, kE8M0One, 0, kE8M0One);
            if (split) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[i][j][r] = __builtin_fmaf(P[r] * sr.sa[i], cv[j][r], acc[i][j][r]);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(P[r], s[i], acc[i][j][r]);
            }
          }
        }
      }
    };

    k_loop(group);
    wait_vmcnt<0>();  // no LDS copy may land after the workgroup ends

    // ---- epilogue: lane holds row fr of tile i, columns 4 (l/16) .. +3 of tile j
    if constexpr (CT == 0) {
      const bool vec = p.vec_store != 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + fr;
        if (row >= rows_valid) continue;
        const int64_t grow = row_base + row;
        float rs = 1.0f;
        if constexpr (!kPromote) rs = p.sa[grow * p.sa_ms];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v[r] = acc[i][j][r];
            if constexpr (!kPromote) {
              const float cs = BMODE == 0 ? SB[(n0 >> 7) * p.sb_ns] : SB[(col + r) * p.sb_ns];
              v[r] = v[r] * (rs * cs);
            }
          }
          store_c4<CT>(p.c, grow * p.ldc + col, v, vec);
        }
      }
    } else {
      // FP32 output: one copy of the stores per width, so that the aligned
      // copy keeps its 16-byte stores (with a per-store choice the compiler
      // merges the two forms into narrower ones).
      auto epilogue = [&](auto vec_c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm * 64 + i * 16 + fr;
          if (row >= rows_valid) continue;
          const int64_t grow = row_base + row;
          float rs = 1.0f;
          if constexpr (!kPromote) rs = p.sa[grow * p.sa_ms];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              v[r] = acc[i][j][r];
              if constexpr (!kPromote) {
                const float cs = BMODE == 0 ? SB[(n0 >> 7) * p.sb_ns] : SB[(col + r) * p.sb_ns];
                v[r] = v[r] * (rs * cs);
              }
            }
            store_c4<CT>(p.c, grow * p.ldc + col, v, decltype(vec_c)::value);
          }
        }
      };
      if (p.vec_store != 0)
        epilogue(BoolTag<true>{});
      else
        epilogue(BoolTag<false>{});
    }
  }
}

// ===========================================================================
// Default path (exact partial sums, 128x128 B block scales): rescaled
// accumulation on 256 x (64 JT) tiles, JT = 4 (256 columns) or 3 (192).
//
// The group scale of output element (m, n) is sigma_kb = sa(m, kb) *
// sb(kb, n / 128).  The FP32 accumulator D holds the running sum in units of
// the current group's scale: before the group's products are added (by the
// MFMA itself),
//   D <- D * (sigma_{kb-1} / sigma_kb),
// and the epilogue writes C = sigma_last * D.  This applies every group's
// scales to full FP32 accumulators once per 128 of K, as the separate-P
// form does, with one multiply per element and group, but without a second
// set of accumulators -- which is what makes a 64x(32 JT) wave tile fit.
// The scale is kept as a mantissa product in [0.25, 1) and an exponent
// (the FP32 product of the two scales can be a denormal, which would cost
// precision), and the per-group ratio is formed from them so that nothing
// overflows on the way.  D's units never go below 2^-64 of the largest
// scale taken so far: a group with a smaller scale is accumulated in those
// floor units instead of its own.  Its products then enter with a weight at
// most 2^-64 of that largest scale where the true weight is smaller still,
// so the difference is below 2^-39 of the largest group term; and D stays
// bounded (each group adds less than 2^91 units, so |D| < 2^115 for K < 2^31).
//
// JT = 4: the 128 columns of a wave lie in one B scale block (tiles start at
// multiples of 256), so sigma is one value per lane and row tile.  JT = 3: a
// wave's 96 columns can straddle two B blocks, so sigma is tracked per row
// tile and column tile.
constexpr int kDropExp = 64;  // floor of D's units: 2^-64 of the largest scale taken

template <int JT>
struct __align__(16) Stage2 {
  uint8_t a[kBM * kBK];
  uint8_t b[64 * JT * kBK];
};


template <int CT, int JT>
__global__ __launch_bounds__(kThreads, 1) void gemm_rescale_kernel(KParams p) {
  constexpr int kBNT = 64 * JT;         // workgroup tile columns
  constexpr int kWN = 32 * JT;          // wave tile columns
  constexpr bool kPerJ = JT != 4;
  constexpr int kDmaA = kBM / (8 * kWaves);
  constexpr int kDmaB = kBNT / (8 * kWaves);
  // Two stages, each its own LDS object (the K loop is unrolled by two).
  __shared__ Stage2<JT> stage0;
  __shared__ Stage2<JT> stage1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave >> 1;  // rows wm*64 .. +64
  const int wn = wave & 1;   // columns wn*kWN .. +kWN

  // ---- tile decode
  const int id = tile_id<false>(p, kBM);
  if (id < 0) return;
  const uint8_t* A = p.a;
  const uint8_t* B = p.b;
  const float* SB = p.sb;
  int64_t row_base = 0;
  int rows_valid = 0;
  int tn = 0;
  {
    const int tiles_m = (int)((p.M + kBM - 1) / kBM);
    int tm;
    grouped_order(id, tiles_m, p.tiles_n, tm, tn);
    row_base = (int64_t)tm * kBM;
    const int64_t rem = p.M - row_base;
    rows_valid = rem < kBM ? (int)rem : kBM;
  }
  const int64_t n0 = p.n_base + (int64_t)tn * kBNT;
  const int nkb = (int)(p.K / kBK);

  // ---- copy sources: instruction i of wave w fills LDS rows (8i + w) * 8 .. +8
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + row_base * p.lda, (uint32_t)(rows_valid * p.lda));
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + n0 * p.ldb, (uint32_t)(kBNT * p.ldb));
  const __amdgpu_buffer_rsrc_t null_rsrc = make_rsrc(p.a, 0u);
  uint32_t a_off[kDmaA], b_off[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    const int ra = r < rows_valid ? r : rows_valid - 1;  // ragged M: repeat the last row
    a_off[i] = (uint32_t)(ra * p.lda + (((lane & 7) ^ swz(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    b_off[i] = (uint32_t)(r * p.ldb + (((lane & 7) ^ swz(r)) << 4));
  }
  // Every group issues the same copies (empty ones past the last group).
  auto issue = [&](int kb, Stage2<JT>& S) {
    const bool live = kb < nkb;
    const uint32_t koff = live ? (uint32_t)kb * kBK : 0u;
    const __amdgpu_buffer_rsrc_t ra = live ? a_rsrc : null_rsrc;
    const __amdgpu_buffer_rsrc_t rb = live ? b_rsrc : null_rsrc;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) dma16(ra, a_off[i], koff, S.a + (i * kWaves + wave) * 1024);
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) dma16(rb, b_off[i], koff, S.b + (i * kWaves + wave) * 1024);
  };

  // ---- scale sources: this lane's output row in row tile i is wm*64 + i*32 + lane % 32;
  // column tile j of the wave lies in B scale block (n0 + wn*kWN + 32 j) / 128
  const int g = lane >> 5;
  const int lr = lane & 31;
  constexpr int NB = kPerJ ? JT : 1;  // B scales per group and wave
  const __amdgpu_buffer_rsrc_t sa_rsrc = make_rsrc(p.sa + row_base * p.sa_ms, 0xFFFFFFFFu);
  uint32_t sa_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wm * 64 + i * 32 + lr;
    sa_off[i] = (uint32_t)((r < rows_valid ? r : rows_valid - 1) * p.sa_ms * 4);
  }
  __amdgpu_buffer_rsrc_t sb_rsrc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
    sb_rsrc[j] = make_rsrc(SB + ((n0 + wn * kWN + 32 * j) >> 7) * p.sb_ns, 0xFFFFFFFFu);
  struct ScaleRegs {
    float sa[2];
    float sb[NB];
  };
  auto load_scales = [&](int kb, ScaleRegs& s) {
    const bool live = kb < nkb;
    const __amdgpu_buffer_rsrc_t ra = live ? sa_rsrc : null_rsrc;
    const uint32_t ka = live ? (uint32_t)(kb * p.sa_ks * 4) : 0u;
    const uint32_t kbo = live ? (uint32_t)(kb * p.sb_ks * 4) : 0u;
#pragma unroll
    for (int i = 0; i < 2; ++i) s.sa[i] = load_f32(ra, sa_off[i], ka);
#pragma unroll
    for (int j = 0; j < NB; ++j) s.sb[j] = load_f32(live ? sb_rsrc[j] : null_rsrc, 0u, kbo);
  };

  // Wave tile 64 x kWN = 2 x JT tiles of 32x32.  B is the first MFMA operand,
  // so accumulator element r of lane l is row lr of row tile i and column
  // 8 (r / 4) + 4 g + r % 4 of column tile j.
  v16f D[2][JT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) D[i][j][r] = 0.f;
  // D of (row tile i, scale column c) is expressed in units of
  // mc * 2^ec, split into a mantissa in [0.25, 1] and an exponent; mc = 0
  // before anything was accumulated.  emax is the largest exponent of a
  // scale product taken so far.  c = j when scales differ per column tile,
  // else 0.
  float mc[2][NB], rs[2][NB];
  int ec[2][NB], emax[2][NB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      mc[i][j] = 0.f;
      rs[i][j] = 1.f;
      ec[i][j] = 0;
      emax[i][j] = -(1 << 20);
    }

  // Top of group kb (team 0; team 1 waits at its step 4, see the group
  // below): the copies issued in group kb - 1 (this group's data) are the
  // newest memory operations, so wait for all; after the barrier every
  // wave's copies of this group have landed and every wave has finished
  // reading the other stage.
  auto wait_group = [&]() {
    wait_vmcnt<0>();
    block_barrier();
  };

  // Rescale factors of a group: rs = (mc / m) * 2^(ec - e) for the group's
  // scale product m * 2^e; the mantissa quotient lies in (0.25, 4), so
  // nothing overflows before the exponent is applied (the reciprocal is
  // refined by one Newton step).  Computed at the end of the previous group,
  // off the critical path.
  auto factors = [&](const ScaleRegs& sr) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float a = sr.sa[i];
      const float ma = __builtin_amdgcn_frexp_mantf(a);
      const int ea = __builtin_amdgcn_frexp_expf(a);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float b = sr.sb[j];
        float m = ma * __builtin_amdgcn_frexp_mantf(b);
        int e = ea + __builtin_amdgcn_frexp_expf(b);
        // below the floor (or a zero scale): accumulate in the floor units
        const bool low = a == 0.f || b == 0.f || e < emax[i][j] - kDropExp;
        m = low ? 1.0f : m;
        e = low ? emax[i][j] - kDropExp : e;
        float r = __builtin_amdgcn_rcpf(m);
        r = __builtin_fmaf(__builtin_fmaf(-m, r, 1.0f), r, r);
        rs[i][j] = __builtin_amdgcn_ldexpf(mc[i][j] * r, ec[i][j] - e);
        mc[i][j] = m;
        ec[i][j] = e;
        emax[i][j] = e > emax[i][j] ? e : emax[i][j];
      }
    }
  };

  auto cvt8 = [](uint32_t lo, uint32_t hi, float sc) {
    union {
      v2bf p[4];
      v8bf v;
    } u;
    u.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, sc, false);
    u.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, sc, true);
    u.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, sc, false);
    u.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, sc, true);
    return u.v;
  };

  // Group kb loads the scales of group kb + 2 into the register set that
  // held group kb's (consumed at the end of group kb - 1), and at its end
  // forms the factors of group kb + 1 from scales loaded a group earlier.
  //
  // Two teams, one wave of each on every SIMD (waves w and w + 4 share a
  // SIMD): team 0 takes the group's barrier at the top of the group and then
  // issues the next group's copies; team 1 takes it after step 4, where it
  // has read its last chunk of the group, and then issues the copies of the
  // group after next into the stage it has just finished reading.  So team 1
  // runs three K steps behind team 0, and on each SIMD one wave's group
  // prologue (fragment reads, rescale multiplies, first conversions, with no
  // MFMA of its own in flight) meets the other wave's MFMA steps.  Every
  // barrier pairs the two teams' positions: a stage is refilled only after
  // both have read it, and each copy still has one group's time to land.
  auto group = [&](auto team_tag, int kb, const Stage2<JT>& S, Stage2<JT>& Nx, ScaleRegs& lsr,
                   const ScaleRegs& fsr) {
    constexpr int kTeam = decltype(team_tag)::value;
    if constexpr (kTeam == 0) wait_group();
    uint4 ra[4][2], rb[4][JT];
    auto read_chunk = [&](int c) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + lr;
        ra[c][i] = *reinterpret_cast<const uint4*>(S.a + row * 128 + (((4 * g + c) ^ swz(row)) << 4));
      }
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const int row = wn * kWN + j * 32 + lr;
        rb[c][j] = *reinterpret_cast<const uint4*>(S.b + row * 128 + (((4 * g + c) ^ swz(row)) << 4));
      }
    };
    v8bf af[2][2], bfr[2][JT];  // [step parity][tile]
    auto convert = [&](int st) {
      const int c = st >> 1, h = st & 1, par = st & 1;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[par][i] = h ? cvt8(ra[c][i].z, ra[c][i].w, 1.0f) : cvt8(ra[c][i].x, ra[c][i].y, 1.0f);
#pragma unroll
      for (int j = 0; j < JT; ++j)
        bfr[par][j] = h ? cvt8(rb[c][j].z, rb[c][j].w, 1.0f) : cvt8(rb[c][j].x, rb[c][j].y, 1.0f);
    };
    read_chunk(0);
    read_chunk(1);
    __builtin_amdgcn_sched_barrier(0);
    // scales of group kb + 2; team 0: copies of group kb + 1 (into the other stage)
    load_scales(kb + 2, lsr);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kTeam == 0) {
      issue(kb + 1, Nx);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the rescale runs while the fragment reads are in flight
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) D[i][j][r] *= rs[i][kPerJ ? j : 0];
    convert(0);
    __builtin_amdgcn_sched_barrier(0);
    // Raised wave priority while the MFMA steps run: the wave in its MFMA
    // steps issues first, and the other wave of the SIMD, in its prologue,
    // fills in (with the teams staggered, 12% faster than without it).
    __builtin_amdgcn_s_setprio(1);
    // the 8 K steps
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int par = st & 1;
      // chunk c + 1 is read at step 2c, one step before its first conversion
      if (!(st & 1) && st >= 2 && (st >> 1) + 1 < 4) read_chunk((st >> 1) + 1);
      if (st + 1 < 8) convert(st + 1);
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          D[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[par][j], af[par][i], D[i][j], 0, 0, 0);
      if (!(st & 1) && st >= 2 && (st >> 1) + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2 + JT, 0);
#pragma unroll
      for (int m = 0; m < 2 * JT; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (st + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kTeam == 1) {
        if (st == 4) {
          // This group's last chunk was read at this step.  Its LDS reads
          // must have returned before the barrier: after it, team 0 refills
          // the stage they read.
          wait_copies_and_reads();
          block_barrier();
          issue(kb + 2, const_cast<Stage2<JT>&>(S));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // the next group's factors, while this group's last MFMAs run (none
    // after the last group: the epilogue needs this group's units)
    if (kb + 1 < nkb) factors(fsr);
  };

  ScaleRegs sr0{}, sr1{};
  load_scales(0, sr0);
  load_scales(1, sr1);
  issue(0, stage0);
  factors(sr0);
  // every wave's copies of group 0 have landed after this barrier
  wait_vmcnt<0>();
  block_barrier();
  // Barriers: team 0 takes one at the top of each group and one at the end,
  // team 1 one at the start and one in each group, nkb + 1 each.
  if ((wave >> 2) == 0) {
    int kb = 0;
    for (; kb + 2 <= nkb; kb += 2) {
      group(IntTag<0>{}, kb, stage0, stage1, sr0, sr1);
      group(IntTag<0>{}, kb + 1, stage1, stage0, sr1, sr0);
    }
    if (kb < nkb) group(IntTag<0>{}, kb, stage0, stage1, sr0, sr1);
    wait_vmcnt<0>();
    block_barrier();  // with team 1's in its last group
  } else {
    block_barrier();  // with team 0's at the top of group 0
    issue(1, stage1);
    int kb = 0;
    for (; kb + 2 <= nkb; kb += 2) {
      group(IntTag<1>{}, kb, stage0, stage1, sr0, sr1);
      group(IntTag<1>{}, kb + 1, stage1, stage0, sr1, sr0);
    }
    if (kb < nkb) group(IntTag<1>{}, kb, stage0, stage1, sr0, sr1);
  }
  wait_vmcnt<0>();  // no LDS copy may land after the workgroup ends

  // ---- epilogue: C = D * mc * 2^ec; lane holds row lr of row tile i,
  // columns 8q + 4g .. +3 of column tile j
  if constexpr (CT == 0) {
    const bool vec = p.vec_store != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + i * 32 + lr;
      if (row >= rows_valid) continue;
      const int64_t grow = row_base + row;
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = n0 + wn * kWN + j * 32 + 8 * q + 4 * g;
          const int c = kPerJ ? j : 0;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = __builtin_amdgcn_ldexpf(D[i][j][4 * q + t] * mc[i][c], ec[i][c]);
          store_c4<CT>(p.c, grow * p.ldc + col, v, vec);
        }
    }
  } else {
    // FP32 output: one copy of the stores per width, so that the aligned
    // copy keeps its 16-byte stores (with a per-store choice the compiler
    // merges the two forms into narrower ones).
    auto epilogue = [&](auto vec_c) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + lr;
        if (row >= rows_valid) continue;
        const int64_t grow = row_base + row;
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t col = n0 + wn * kWN + j * 32 + 8 * q + 4 * g;
            const int c = kPerJ ? j : 0;
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = __builtin_amdgcn_ldexpf(D[i][j][4 * q + t] * mc[i][c], ec[i][c]);
            store_c4<CT>(p.c, grow * p.ldc + col, v, decltype(vec_c)::value);
          }
      }
    };
    if (p.vec_store != 0)
      epilogue(BoolTag<true>{});
    else
      epilogue(BoolTag<false>{});
  }
}


// Tile of a grouped launch of the rescaled-accumulation kernel.  Each
// expert's rows are cut into 256-row tiles, except that a last tile of at
// most 128 rows is a 128-row tile (half the work of a 256-row one).  The
// 256-row tiles of all experts take workgroups 0 .. nbig - 1 (renumbered
// over the XCDs as in tile_id); the 128-row tiles take the workgroups from
// the next multiple of 8 on, so that every XCD runs its share of them after
// its 256-row tiles.  The launch holds at least ceil(M / 256) + G row tiles
// of workgroups plus 7; those without a tile return false.
__device__ __forceinline__ bool grouped_rescale_tile(const KParams& p, int& expert, int64_t& row_base,
                                                     int& rows_valid, int& tn, bool& half) {
  int nbig = 0, nhalf = 0;
  for (int e = 0; e < p.G; ++e) {
    const int64_t rows = (int64_t)p.offsets[e + 1] - p.offsets[e];
    const int64_t tail = rows % kBM;
    nbig += (int)(rows / kBM) + (tail > kBM / 2 ? 1 : 0);
    nhalf += tail > 0 && tail <= kBM / 2 ? 1 : 0;
  }
  nbig *= p.tiles_n;
  nhalf *= p.tiles_n;
  const int big_end = (nbig + 7) & ~7;
  const int b = (int)blockIdx.x;
  int t;
  if (b < nbig) {
    half = false;
    t = xcd_remap(b, nbig);
  } else if (b >= big_end && b - big_end < nhalf) {
    half = true;
    t = xcd_remap(b - big_end, nhalf);  // big_end % 8 == 0: same XCD as b
  } else {
    return false;
  }
  for (int e = 0; e < p.G; ++e) {
    const int64_t seg0 = p.offsets[e];
    const int64_t seg1 = p.offsets[e + 1];
    const int64_t rows = seg1 - seg0;
    const int64_t tail = rows % kBM;
    if (!half) {
      const int tm_e = (int)(rows / kBM) + (tail > kBM / 2 ? 1 : 0);
      const int cnt = tm_e * p.tiles_n;
      if (t < cnt) {
        int tm;
        grouped_order(t, tm_e, p.tiles_n, tm, tn);
        row_base = seg0 + (int64_t)tm * kBM;
        const int64_t rem = seg1 - row_base;
        rows_valid = rem < kBM ? (int)rem : kBM;
        expert = e;
        return true;
      }
      t -= cnt;
    } else if (tail > 0 && tail <= kBM / 2) {
      if (t < p.tiles_n) {
        tn = t;
        row_base = seg1 - tail;
        rows_valid = (int)tail;
        expert = e;
        return true;
      }
      t -= p.tiles_n;
    }
  }
  return false;
}

// The grouped form of gemm_rescale_kernel: the same arithmetic per output
// element, on 256-row tiles plus the 128-row tiles that end experts with at
// most 128 rows left (RT row tiles of 32 per wave, chosen per workgroup).
// It is a kernel of its own because the form with two tile heights in one
// kernel runs 1-3% slower on dense shapes, where it is never needed.
template <int CT, int JT>
__global__ __launch_bounds__(kThreads, 1) void gemm_rescale_grouped_kernel(KParams p) {
  constexpr int kBNT = 64 * JT;         // workgroup tile columns
  constexpr int kWN = 32 * JT;          // wave tile columns
  constexpr bool kPerJ = JT != 4;
  constexpr int kDmaB = kBNT / (8 * kWaves);
  // Two stages, the A and B parts of each their own LDS object (the K loop
  // is unrolled by two).  With one object per stage, the pointer chains of
  // the B fragment reads grow past the depth at which the compiler keeps
  // their LDS alias scopes, and every group then waits for the next group's
  // copies before those reads.
  __shared__ __align__(16) uint8_t s0a[kBM * kBK];
  __shared__ __align__(16) uint8_t s0b[kBNT * kBK];
  __shared__ __align__(16) uint8_t s1a[kBM * kBK];
  __shared__ __align__(16) uint8_t s1b[kBNT * kBK];
  struct StageRef {
    uint8_t* a;
    uint8_t* b;
  };
  const StageRef stage0{s0a, s0b}, stage1{s1a, s1b};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave >> 1;  // row group of the wave
  const int wn = wave & 1;   // columns wn*kWN .. +kWN

  // ---- tile decode
  const uint8_t* A = p.a;
  const uint8_t* B = p.b;
  const float* SB = p.sb;
  int64_t row_base = 0;
  int rows_valid = 0;
  int tn = 0;
  bool half = false;  // a 128-row tile
  {
    int e = 0;
    if (!grouped_rescale_tile(p, e, row_base, rows_valid, tn, half)) return;
    B += (int64_t)e * p.b_gs;
    SB += (int64_t)e * p.sb_gs;
  }
  const int64_t n0 = p.n_base + (int64_t)tn * kBNT;
  const int nkb = (int)(p.K / kBK);

  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + row_base * p.lda, (uint32_t)(rows_valid * p.lda));
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + n0 * p.ldb, (uint32_t)(kBNT * p.ldb));
  const __amdgpu_buffer_rsrc_t null_rsrc = make_rsrc(p.a, 0u);
  uint32_t b_off[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    b_off[i] = (uint32_t)(r * p.ldb + (((lane & 7) ^ swz(r)) << 4));
  }
  const int g = lane >> 5;
  const int lr = lane & 31;
  constexpr int NB = kPerJ ? JT : 1;  // B scales per group and wave
  const __amdgpu_buffer_rsrc_t sa_rsrc = make_rsrc(p.sa + row_base * p.sa_ms, 0xFFFFFFFFu);
  __amdgpu_buffer_rsrc_t sb_rsrc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
    sb_rsrc[j] = make_rsrc(SB + ((n0 + wn * kWN + 32 * j) >> 7) * p.sb_ns, 0xFFFFFFFFu);

  // The rest is written for RT row tiles of 32 per wave: RT = 2 on 256-row
  // tiles (wave rows wm*64 .. +64), RT = 1 on 128-row tiles (wm*32 .. +32).
  // Every 32x32 output tile sees the same operations in the same order
  // either way.
  auto body = [&](auto rt_c) {
    constexpr int RT = decltype(rt_c)::value;
    constexpr int kDmaA = 32 * RT * 4 / (8 * kWaves);
    // ---- copy sources: instruction i of wave w fills LDS rows (8i + w) * 8 .. +8
    uint32_t a_off[kDmaA];
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) {
      const int r = (i * kWaves + wave) * 8 + (lane >> 3);
      const int ra = r < rows_valid ? r : rows_valid - 1;  // ragged M: repeat the last row
      a_off[i] = (uint32_t)(ra * p.lda + (((lane & 7) ^ swz(r)) << 4));
    }
    // Every group issues the same copies (empty ones past the last group).
    auto issue = [&](int kb, const StageRef& S) {
      const bool live = kb < nkb;
      const uint32_t koff = live ? (uint32_t)kb * kBK : 0u;
      const __amdgpu_buffer_rsrc_t ra = live ? a_rsrc : null_rsrc;
      const __amdgpu_buffer_rsrc_t rb = live ? b_rsrc : null_rsrc;
#pragma unroll
      for (int i = 0; i < kDmaA; ++i) dma16(ra, a_off[i], koff, S.a + (i * kWaves + wave) * 1024);
#pragma unroll
      for (int i = 0; i < kDmaB; ++i) dma16(rb, b_off[i], koff, S.b + (i * kWaves + wave) * 1024);
    };

    // ---- scale sources: this lane's output row in row tile i is
    // wm*32*RT + i*32 + lane % 32; column tile j of the wave lies in B scale
    // block (n0 + wn*kWN + 32 j) / 128
    uint32_t sa_off[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int r = wm * 32 * RT + i * 32 + lr;
      sa_off[i] = (uint32_t)((r < rows_valid ? r : rows_valid - 1) * p.sa_ms * 4);
    }
    struct ScaleRegs {
      float sa[RT];
      float sb[NB];
    };
    auto load_scales = [&](int kb, ScaleRegs& s) {
      const bool live = kb < nkb;
      const __amdgpu_buffer_rsrc_t ra = live ? sa_rsrc : null_rsrc;
      const uint32_t ka = live ? (uint32_t)(kb * p.sa_ks * 4) : 0u;
      const uint32_t kbo = live ? (uint32_t)(kb * p.sb_ks * 4) : 0u;
#pragma unroll
      for (int i = 0; i < RT; ++i) s.sa[i] = load_f32(ra, sa_off[i], ka);
#pragma unroll
      for (int j = 0; j < NB; ++j) s.sb[j] = load_f32(live ? sb_rsrc[j] : null_rsrc, 0u, kbo);
    };

    // Wave tile 32*RT x kWN = RT x JT tiles of 32x32.  B is the first MFMA
    // operand, so accumulator element r of lane l is row lr of row tile i
    // and column 8 (r / 4) + 4 g + r % 4 of column tile j.
    v16f D[RT][JT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) D[i][j][r] = 0.f;
    // D of (row tile i, scale column c) is expressed in units of
    // mc * 2^ec, split into a mantissa in [0.25, 1] and an exponent; mc = 0
    // before anything was accumulated.  emax is the largest exponent of a
    // scale product taken so far.  c = j when scales differ per column tile,
    // else 0.
    float mc[RT][NB], rs[RT][NB];
    int ec[RT][NB], emax[RT][NB];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        mc[i][j] = 0.f;
        rs[i][j] = 1.f;
        ec[i][j] = 0;
        emax[i][j] = -(1 << 20);
      }

    // Top of group kb (team 0; team 1 waits at its step 4): the copies
    // issued in group kb - 1 (this group's data) are the newest memory
    // operations, so wait for all; after the barrier every wave's copies of
    // this group have landed and every wave has finished reading the other
    // stage.
    auto wait_group = [&]() {
      wait_vmcnt<0>();
      block_barrier();
    };

    // Rescale factors of a group: rs = (mc / m) * 2^(ec - e) for the group's
    // scale product m * 2^e; the mantissa quotient lies in (0.25, 4), so
    // nothing overflows before the exponent is applied (the reciprocal is
    // refined by one Newton step).  Computed at the end of the previous group,
    // off the critical path.
    auto factors = [&](const ScaleRegs& sr) {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const float a = sr.sa[i];
        const float ma = __builtin_amdgcn_frexp_mantf(a);
        const int ea = __builtin_amdgcn_frexp_expf(a);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const float b = sr.sb[j];
          float m = ma * __builtin_amdgcn_frexp_mantf(b);
          int e = ea + __builtin_amdgcn_frexp_expf(b);
          // below the floor (or a zero scale): accumulate in the floor units
          const bool low = a == 0.f || b == 0.f || e < emax[i][j] - kDropExp;
          m = low ? 1.0f : m;
          e = low ? emax[i][j] - kDropExp : e;
          float r = __builtin_amdgcn_rcpf(m);
          r = __builtin_fmaf(__builtin_fmaf(-m, r, 1.0f), r, r);
          rs[i][j] = __builtin_amdgcn_ldexpf(mc[i][j] * r, ec[i][j] - e);
          mc[i][j] = m;
          ec[i][j] = e;
          emax[i][j] = e > emax[i][j] ? e : emax[i][j];
        }
      }
    };

    auto cvt8 = [](uint32_t lo, uint32_t hi, float sc) {
      union {
        v2bf p[4];
        v8bf v;
      } u;
      u.p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, sc, false);
      u.p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, sc, true);
      u.p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, sc, false);
      u.p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, sc, true);
      return u.v;
    };

    // MFMAs and conversions of one K step, for the schedule hints below
    constexpr int kMfmaPerStep = RT * JT;
    constexpr int kValuPerMfma = 4 * (RT + JT) / kMfmaPerStep;

    // Group kb loads the scales of group kb + 2 into the register set that
    // held group kb's (consumed at the end of group kb - 1), and at its end
    // forms the factors of group kb + 1 from scales loaded a group earlier.
    // The waves form two staggered teams as in gemm_rescale_kernel: team 0
    // (waves 0-3) takes the group's barrier at its top and issues the next
    // group's copies; team 1 (waves 4-7, one on each SIMD beside a team-0
    // wave) takes it after step 4, its last chunk read, and then issues the
    // copies of the group after next into the stage it has finished reading.
    auto group = [&](auto team_tag, int kb, const StageRef& S, const StageRef& Nx, ScaleRegs& lsr,
                     const ScaleRegs& fsr) {
      constexpr int kTeam = decltype(team_tag)::value;
      if constexpr (kTeam == 0) wait_group();
      uint4 ra[4][RT], rb[4][JT];
      auto read_chunk = [&](int c) {
#pragma unroll
        for (int i = 0; i < RT; ++i) {
          const int row = wm * 32 * RT + i * 32 + lr;
          ra[c][i] = *reinterpret_cast<const uint4*>(S.a + row * 128 + (((4 * g + c) ^ swz(row)) << 4));
        }
#pragma unroll
        for (int j = 0; j < JT; ++j) {
          const int row = wn * kWN + j * 32 + lr;
          rb[c][j] = *reinterpret_cast<const uint4*>(S.b + row * 128 + (((4 * g + c) ^ swz(row)) << 4));
        }
      };
      v8bf af[2][RT], bfr[2][JT];  // [step parity][tile]
      auto convert = [&](int st) {
        const int c = st >> 1, h = st & 1, par = st & 1;
#pragma unroll
        for (int i = 0; i < RT; ++i)
          af[par][i] = h ? cvt8(ra[c][i].z, ra[c][i].w, 1.0f) : cvt8(ra[c][i].x, ra[c][i].y, 1.0f);
#pragma unroll
        for (int j = 0; j < JT; ++j)
          bfr[par][j] = h ? cvt8(rb[c][j].z, rb[c][j].w, 1.0f) : cvt8(rb[c][j].x, rb[c][j].y, 1.0f);
      };
      read_chunk(0);
      read_chunk(1);
      __builtin_amdgcn_sched_barrier(0);
      // scales of group kb + 2; team 0: copies of group kb + 1 (into the other stage)
      load_scales(kb + 2, lsr);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kTeam == 0) {
        issue(kb + 1, Nx);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the rescale runs while the fragment reads are in flight
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) D[i][j][r] *= rs[i][kPerJ ? j : 0];
      convert(0);
      __builtin_amdgcn_sched_barrier(0);
      // the 8 K steps
      auto steps = [&]() {
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int par = st & 1;
          // chunk c + 1 is read at step 2c, one step before its first conversion
          if (!(st & 1) && st >= 2 && (st >> 1) + 1 < 4) read_chunk((st >> 1) + 1);
          if (st + 1 < 8) convert(st + 1);
#pragma unroll
          for (int j = 0; j < JT; ++j)
#pragma unroll
            for (int i = 0; i < RT; ++i)
              D[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[par][j], af[par][i], D[i][j], 0, 0, 0);
          if (!(st & 1) && st >= 2 && (st >> 1) + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, RT + JT, 0);
#pragma unroll
          for (int m = 0; m < kMfmaPerStep; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (st + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kTeam == 1) {
            if (st == 4) {
              // this group's last chunk was read at this step; its LDS
              // reads return before the barrier (team 0 then refills the stage)
              wait_copies_and_reads();
              block_barrier();
              issue(kb + 2, S);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      };
      // Raised wave priority while the MFMA steps run: the wave in its MFMA
      // steps issues first, and the other wave of the SIMD, in its prologue,
      // fills in.
      __builtin_amdgcn_s_setprio(1);
      steps();
      __builtin_amdgcn_s_setprio(0);
      // the next group's factors, while this group's last MFMAs run (none
      // after the last group: the epilogue needs this group's units)
      if (kb + 1 < nkb) factors(fsr);
    };

    // The kernel arguments that only the epilogue reads are made to arrive
    // before the K loop.  Scalar and LDS loads share one counter and scalar
    // loads complete out of order, so one still in flight at the loop entry
    // would turn the first fragment wait of every group into a full drain.
    asm volatile("" ::"s"(p.c), "s"(p.ldc), "s"(p.vec_store));
    ScaleRegs sr0{}, sr1{};
    load_scales(0, sr0);
    load_scales(1, sr1);
    issue(0, stage0);
    factors(sr0);
    // every wave's copies of group 0 have landed after this barrier
    wait_vmcnt<0>();
    block_barrier();
    // Barriers: team 0 takes one at the top of each group and one at the
    // end, team 1 one at the start and one in each group, nkb + 1 each.
    if ((wave >> 2) == 0) {
      int kb = 0;
      for (; kb + 2 <= nkb; kb += 2) {
        group(IntTag<0>{}, kb, stage0, stage1, sr0, sr1);
        group(IntTag<0>{}, kb + 1, stage1, stage0, sr1, sr0);
      }
      if (kb < nkb) group(IntTag<0>{}, kb, stage0, stage1, sr0, sr1);
      wait_vmcnt<0>();
      block_barrier();  // with team 1's in its last group
    } else {
      block_barrier();  // with team 0's at the top of group 0
      issue(1, stage1);
      int kb = 0;
      for (; kb + 2 <= nkb; kb += 2) {
        group(IntTag<1>{}, kb, stage0, stage1, sr0, sr1);
        group(IntTag<1>{}, kb + 1, stage1, stage0, sr1, sr0);
      }
      if (kb < nkb) group(IntTag<1>{}, kb, stage0, stage1, sr0, sr1);
    }
    wait_vmcnt<0>();  // no LDS copy may land after the workgroup ends

    // ---- epilogue: C = D * mc * 2^ec; lane holds row lr of row tile i,
    // columns 8q + 4g .. +3 of column tile j
    if constexpr (CT == 0) {
      const bool vec = p.vec_store != 0;
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int row = wm * 32 * RT + i * 32 + lr;
        if (row >= rows_valid) continue;
        const int64_t grow = row_base + row;
#pragma unroll
        for (int j = 0; j < JT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t col = n0 + wn * kWN + j * 32 + 8 * q + 4 * g;
            const int c = kPerJ ? j : 0;
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = __builtin_amdgcn_ldexpf(D[i][j][4 * q + t] * mc[i][c], ec[i][c]);
            store_c4<CT>(p.c, grow * p.ldc + col, v, vec);
          }
      }
    } else {
      // FP32 output: one copy of the stores per width, so that the aligned
      // copy keeps its 16-byte stores (with a per-store choice the compiler
      // merges the two forms into narrower ones).
      auto epilogue = [&](auto vec_c) {
#pragma unroll
        for (int i = 0; i < RT; ++i) {
          const int row = wm * 32 * RT + i * 32 + lr;
          if (row >= rows_valid) continue;
          const int64_t grow = row_base + row;
#pragma unroll
          for (int j = 0; j < JT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t col = n0 + wn * kWN + j * 32 + 8 * q + 4 * g;
              const int c = kPerJ ? j : 0;
              float v[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) v[t] = __builtin_amdgcn_ldexpf(D[i][j][4 * q + t] * mc[i][c], ec[i][c]);
              store_c4<CT>(p.c, grow * p.ldc + col, v, decltype(vec_c)::value);
            }
        }
      };
      if (p.vec_store != 0)
        epilogue(BoolTag<true>{});
      else
        epilogue(BoolTag<false>{});
    }
  };

  if (__builtin_amdgcn_readfirstlane((int)half))
    body(IntTag<1>{});
  else
    body(IntTag<2>{});
}

// ===========================================================================
// Weight-streaming path (few rows per expert, as in MoE decode): the weights
// are nearly all of the bytes and each is used by one row tile only, so the
// kernel is bound by HBM, not by the matrix cores.  Tile 64 (M) x 32*SW (N);
// SW waves, each 64 x 32 (two 32x32 row tiles, one column tile, so one B
// scale block per wave).  The K groups stream through a ring of S LDS
// stages, S - 1 of them in flight.  Every output element sees the same
// operations in the same order as in gemm_rescale_kernel: the same K split
// over lanes and steps, the same BF16 MFMAs, the same per-group rescale of D
// with the 2^-64 floor, and the same epilogue; the results are identical.
constexpr int kWBM = 64;  // rows per tile
// grouped GEMMs with at most this many rows per expert on average stream
constexpr int kStreamRowsPerExpert = 64;
// 4 waves (128 columns) and a 3-stage ring: 72 KB of LDS, two workgroups
// per CU.  Measured on 16 experts x ~32 tokens, 7168 -> 4096: 8 waves (one
// workgroup per CU) with 3 or 4 stages, 4 waves with 2 or 4 stages, and 2
// waves with 2 or 3 stages all stream slower.
constexpr int kStreamWaves = 4;
constexpr int kStreamStages = 3;
constexpr int kStreamGroups = 1;  // K groups per stage

// One stage holds KG consecutive K groups of the tile: rows of 128 KG bytes.
template <int SW, int KG>
struct __align__(16) StageW {
  uint8_t a[kWBM * kBK * KG];
  uint8_t b[32 * SW * kBK * KG];
};

// 16-byte chunk c of row r sits at chunk c ^ swz_w(r): with 128-byte rows as
// in the tiled kernels, with 256-byte rows over all 16 chunks of the row, so
// that 16 consecutive rows read at one logical chunk cover all 64 banks.
template <int KG>
__device__ __forceinline__ int swz_w(int row) {
  return KG == 1 ? swz(row) : (row & 15);
}

// Workgroups per CU that the LDS ring allows (the register budget follows).
template <int SW, int S, int KG>
constexpr int stream_blocks_per_cu() {
  return (160 * 1024) / (S * (int)sizeof(StageW<SW, KG>));
}

template <int CT, bool GROUPED, int SW, int S, int KG>
__global__ __launch_bounds__(64 * SW, (stream_blocks_per_cu<SW, S, KG>())) void gemm_stream_kernel(KParams p) {
  static_assert(S >= 2 && S <= 4, "two to four stages");
  static_assert(KG == 1 || KG == 2, "one or two K groups per stage");
  constexpr int kBNT = 32 * SW;
  constexpr int kRow = kBK * KG;         // bytes per LDS row
  constexpr int kRowsPerCopy = 1024 / kRow;
  constexpr int kChunks = kRow / 16;     // 16-byte chunks per row
  constexpr int kDmaA = kWBM * kRow / (1024 * SW);
  constexpr int kDmaB = kBNT * kRow / (1024 * SW);
  static_assert(kDmaA >= 1 && kDmaA * 1024 * SW == kWBM * kRow, "A copies per wave");
  // vector-memory instructions per wave and stage: copies plus (2 + 1) scale loads per group
  constexpr int kVmPerStage = kDmaA + kDmaB + 3 * KG;
  using Stage = StageW<SW, KG>;
  // One LDS object per stage (the K loop is unrolled by S), so the
  // compiler's wait analysis sees which copies each read depends on.
  __shared__ Stage st0;
  __shared__ Stage st1;
  __shared__ Stage st2;  // S >= 3
  __shared__ Stage st3;  // S == 4

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // column tile of this wave

  // ---- tile decode: logical id -> (expert, row tile, column tile), row tiles fastest
  const int id = tile_id<GROUPED>(p, kWBM);
  if (id < 0) return;
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
      const int tm_e = (int)((seg1 - seg0 + kWBM - 1) / kWBM);
      const int cnt = tm_e * p.tiles_n;
      if (t < cnt) {
        const int tm = t % tm_e;
        tn = t / tm_e;
        row_base = seg0 + (int64_t)tm * kWBM;
        const int64_t rem = seg1 - row_base;
        rows_valid = rem < kWBM ? (int)rem : kWBM;
        found = true;
        break;
      }
      t -= cnt;
    }
    if (!found) return;
    B += (int64_t)e * p.b_gs;
    SB += (int64_t)e * p.sb_gs;
  } else {
    const int tiles_m = (int)((p.M + kWBM - 1) / kWBM);
    const int tm = id % tiles_m;
    tn = id / tiles_m;
    row_base = (int64_t)tm * kWBM;
    const int64_t rem = p.M - row_base;
    rows_valid = rem < kWBM ? (int)rem : kWBM;
  }
  const int64_t n0 = p.n_base + (int64_t)tn * kBNT;
  const int nkb = (int)(p.K / kBK);
  const int nst = (nkb + KG - 1) / KG;  // stages of KG groups

  // ---- copy sources: instruction i of wave w fills LDS rows (i * SW + w) * kRowsPerCopy .. + kRowsPerCopy
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + row_base * p.lda, (uint32_t)(rows_valid * p.lda));
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + n0 * p.ldb, (uint32_t)(kBNT * p.ldb));
  const __amdgpu_buffer_rsrc_t null_rsrc = make_rsrc(p.a, 0u);
  uint32_t a_off[kDmaA], b_off[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int r = (i * SW + wave) * kRowsPerCopy + lane / kChunks;
    const int ra = r < rows_valid ? r : rows_valid - 1;  // ragged M: repeat the last row
    a_off[i] = (uint32_t)(ra * p.lda + (((lane % kChunks) ^ swz_w<KG>(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int r = (i * SW + wave) * kRowsPerCopy + lane / kChunks;
    b_off[i] = (uint32_t)(r * p.ldb + (((lane % kChunks) ^ swz_w<KG>(r)) << 4));
  }

  // ---- scale sources: this lane's output row in row tile i is i*32 + lane % 32;
  // the wave's 32 columns lie in B scale block (n0 + 32 wave) / 128
  const int g = lane >> 5;
  const int lr = lane & 31;
  const __amdgpu_buffer_rsrc_t sa_rsrc = make_rsrc(p.sa + row_base * p.sa_ms, 0xFFFFFFFFu);
  uint32_t sa_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = i * 32 + lr;
    sa_off[i] = (uint32_t)((r < rows_valid ? r : rows_valid - 1) * p.sa_ms * 4);
  }
  const __amdgpu_buffer_rsrc_t sb_rsrc = make_rsrc(SB + ((n0 + 32 * wave) >> 7) * p.sb_ns, 0xFFFFFFFFu);
  struct ScaleRegs {
    float sa[KG][2];
    float sb[KG];
  };

  // Stage sx's scales and copies (groups KG sx ..), all of them empty past
  // the last group so that every stage issues the same instructions.  With
  // KG = 2 and an odd group count the last stage copies 256 bytes per row
  // of which the second half lies past K: the buffer range check returns
  // zeros there, and that group is never computed.
  auto issue = [&](int sx, Stage& Sx, ScaleRegs& sr) {
#pragma unroll
    for (int h = 0; h < KG; ++h) {
      const int kb = KG * sx + h;
      const bool live = kb < nkb;
      const __amdgpu_buffer_rsrc_t rsa = live ? sa_rsrc : null_rsrc;
      const __amdgpu_buffer_rsrc_t rsb = live ? sb_rsrc : null_rsrc;
      const uint32_t ka = live ? (uint32_t)(kb * p.sa_ks * 4) : 0u;
      const uint32_t kbo = live ? (uint32_t)(kb * p.sb_ks * 4) : 0u;
#pragma unroll
      for (int i = 0; i < 2; ++i) sr.sa[h][i] = load_f32(rsa, sa_off[i], ka);
      sr.sb[h] = load_f32(rsb, 0u, kbo);
    }
    const bool live = sx < nst;
    const uint32_t koff = live ? (uint32_t)sx * kRow : 0u;
    const __amdgpu_buffer_rsrc_t ra = live ? a_rsrc : null_rsrc;
    const __amdgpu_buffer_rsrc_t rb = live ? b_rsrc : null_rsrc;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) dma16(ra, a_off[i], koff, Sx.a + (i * SW + wave) * 1024);
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) dma16(rb, b_off[i], koff, Sx.b + (i * SW + wave) * 1024);
  };

  v16f D[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) D[i][r] = 0.f;
  // units of D per row tile: mc * 2^ec; emax: largest scale exponent taken
  float mc[2] = {0.f, 0.f};
  int ec[2] = {0, 0};
  int emax[2] = {-(1 << 20), -(1 << 20)};

  // K group h of the stage Sc: factors, rescale of D and the 8 K steps
  auto compute = [&](int h, const Stage& Sc, const ScaleRegs& src) {
    // factors of this group and the rescale of D (same arithmetic as gemm_rescale_kernel)
    float rs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float a = src.sa[h][i];
      const float b = src.sb[h];
      float m = __builtin_amdgcn_frexp_mantf(a) * __builtin_amdgcn_frexp_mantf(b);
      int e = __builtin_amdgcn_frexp_expf(a) + __builtin_amdgcn_frexp_expf(b);
      const bool low = a == 0.f || b == 0.f || e < emax[i] - kDropExp;
      m = low ? 1.0f : m;
      e = low ? emax[i] - kDropExp : e;
      float r = __builtin_amdgcn_rcpf(m);
      r = __builtin_fmaf(__builtin_fmaf(-m, r, 1.0f), r, r);
      rs[i] = __builtin_amdgcn_ldexpf(mc[i] * r, ec[i] - e);
      mc[i] = m;
      ec[i] = e;
      emax[i] = e > emax[i] ? e : emax[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) D[i][r] *= rs[i];
    // lane half g holds K bytes 64 g .. 64 g + 63 of the group in four
    // 16-byte chunks; step st multiplies bytes 64 g + 8 st .. + 7
    uint4 ra[4][2], rb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = i * 32 + lr;
        ra[c][i] = *reinterpret_cast<const uint4*>(Sc.a + row * kRow + (((8 * h + 4 * g + c) ^ swz_w<KG>(row)) << 4));
      }
      const int row = wave * 32 + lr;
      rb[c] = *reinterpret_cast<const uint4*>(Sc.b + row * kRow + (((8 * h + 4 * g + c) ^ swz_w<KG>(row)) << 4));
    }
#pragma unroll
    for (int stp = 0; stp < 8; ++stp) {
      const int c = stp >> 1;
      const bool hi = stp & 1;
      const v8bf bf = hi ? fp8x8_to_bf16(rb[c].z, rb[c].w) : fp8x8_to_bf16(rb[c].x, rb[c].y);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v8bf af = hi ? fp8x8_to_bf16(ra[c][i].z, ra[c][i].w) : fp8x8_to_bf16(ra[c][i].x, ra[c][i].y);
        D[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, D[i], 0, 0, 0);
      }
    }
  };

  auto stage = [&](int sx, const Stage& Sc, Stage& Sr, const ScaleRegs& src, ScaleRegs& srr) {
    // this stage's copies and scales are older than the S - 2 stages issued since
    wait_vmcnt<(S - 2) * kVmPerStage>();
    block_barrier();
    issue(sx + S - 1, Sr, srr);  // into the stage every wave finished reading last time
    compute(0, Sc, src);
    if constexpr (KG == 2) {
      if (KG * sx + 1 < nkb) compute(1, Sc, src);
    }
  };

  ScaleRegs r0{}, r1{}, r2{}, r3{};
  issue(0, st0, r0);
  int sx = 0;
  if constexpr (S == 2) {
    for (; sx + 2 <= nst; sx += 2) {
      stage(sx, st0, st1, r0, r1);
      stage(sx + 1, st1, st0, r1, r0);
    }
    if (sx < nst) stage(sx, st0, st1, r0, r1);
  } else if constexpr (S == 3) {
    issue(1, st1, r1);
    for (; sx + 3 <= nst; sx += 3) {
      stage(sx, st0, st2, r0, r2);
      stage(sx + 1, st1, st0, r1, r0);
      stage(sx + 2, st2, st1, r2, r1);
    }
    if (sx < nst) stage(sx, st0, st2, r0, r2);
    if (sx + 1 < nst) stage(sx + 1, st1, st0, r1, r0);
  } else {
    issue(1, st1, r1);
    issue(2, st2, r2);
    for (; sx + 4 <= nst; sx += 4) {
      stage(sx, st0, st3, r0, r3);
      stage(sx + 1, st1, st0, r1, r0);
      stage(sx + 2, st2, st1, r2, r1);
      stage(sx + 3, st3, st2, r3, r2);
    }
    if (sx < nst) stage(sx, st0, st3, r0, r3);
    if (sx + 1 < nst) stage(sx + 1, st1, st0, r1, r0);
    if (sx + 2 < nst) stage(sx + 2, st2, st1, r2, r1);
  }
  wait_vmcnt<0>();  // no LDS copy may land after the workgroup ends

  // ---- epilogue: C = D * mc * 2^ec; lane holds row lr of row tile i,
  // columns 8q + 4g .. +3 of the wave's 32
  if constexpr (CT == 0) {
    const bool vec = p.vec_store != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = i * 32 + lr;
      if (row >= rows_valid) continue;
      const int64_t grow = row_base + row;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + wave * 32 + 8 * q + 4 * g;
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = __builtin_amdgcn_ldexpf(D[i][4 * q + t] * mc[i], ec[i]);
        store_c4<CT>(p.c, grow * p.ldc + col, v, vec);
      }
    }
  } else {
    // FP32 output: one copy of the stores per width, so that the aligned
    // copy keeps its 16-byte stores (with a per-store choice the compiler
    // merges the two forms into narrower ones).
    auto epilogue = [&](auto vec_c) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = i * 32 + lr;
        if (row >= rows_valid) continue;
        const int64_t grow = row_base + row;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = n0 + wave * 32 + 8 * q + 4 * g;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = __builtin_amdgcn_ldexpf(D[i][4 * q + t] * mc[i], ec[i]);
          store_c4<CT>(p.c, grow * p.ldc + col, v, decltype(vec_c)::value);
        }
      }
    };
    if (p.vec_store != 0)
      epilogue(BoolTag<true>{});
    else
      epilogue(BoolTag<false>{});
  }
}

template <int CT, bool GROUPED>
hipError_t launch_stream(const KParams& kp, hipStream_t st) {
  hipLaunchKernelGGL((gemm_stream_kernel<CT, GROUPED, kStreamWaves, kStreamStages, kStreamGroups>), dim3(kp.nblocks),
                     dim3(64 * kStreamWaves), 0, st, kp);
  return hipGetLastError();
}

// ===========================================================================
// E8M0-scale path on 256 x 256 tiles (128x128 B block scales, N % 256 == 0):
// the FP8 operands go to v_mfma_scale_f32_32x32x64_f8f6f4 unconverted, with
// each group's scales split as in MODE 3 of gemm_blockscaled_kernel -- the
// power of two as the instruction's E8M0 operand scale, the rest f (1 for
// power-of-two scales) applied in FP32.  The products always accumulate in
// the instruction itself; the accumulator holds D / u, u the f of the
// current group per lane and row tile, and is multiplied by u / f where a
// group's f differs (the scheme of gemm_rescale_kernel, with the powers of
// two left to the instruction; D = acc * u at the end).  Power-of-two
// scales need no multiply at all.  Eight waves of 64 x 128 (2 x 4 tiles of
// 32 x 32), two LDS stages, copies one group ahead, as in
// gemm_rescale_kernel.  Against MODE 3's 256 x 128 tiles this halves the LDS
// bytes read per MFMA flop and replaces its per-group FMA promotion.
//
// Lane l of an MFMA supplies row l % 32 of its operand and 32 of the 64 K
// bytes (half l / 32); A and B fragments use the same split, so every
// product pairs matching K elements whatever order the instruction sums
// them in, and the lanes of one row share that row's scale.
template <int CT, bool GROUPED>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(KParams p) {
  constexpr int kBNT = 256;
  constexpr int kDmaA = kBM / (8 * kWaves);
  constexpr int kDmaB = kBNT / (8 * kWaves);
  __shared__ Stage2<4> stage0;
  __shared__ Stage2<4> stage1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;  // rows wm*64 .. +64
  const int wn = wave & 1;   // columns wn*128 .. +128

  const int id = tile_id<GROUPED>(p, kBM);
  if (id < 0) return;
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
  const int64_t n0 = (int64_t)tn * kBNT;
  const int nkb = (int)(p.K / kBK);

  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + row_base * p.lda, (uint32_t)(rows_valid * p.lda));
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + n0 * p.ldb, (uint32_t)(kBNT * p.ldb));
  const __amdgpu_buffer_rsrc_t null_rsrc = make_rsrc(p.a, 0u);
  uint32_t a_off[kDmaA], b_off[kDmaB];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    const int ra = r < rows_valid ? r : rows_valid - 1;
    a_off[i] = (uint32_t)(ra * p.lda + (((lane & 7) ^ swz(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int r = (i * kWaves + wave) * 8 + (lane >> 3);
    b_off[i] = (uint32_t)(r * p.ldb + (((lane & 7) ^ swz(r)) << 4));
  }
  auto issue = [&](int kb, Stage2<4>& S) {
    const bool live = kb < nkb;
    const uint32_t koff = live ? (uint32_t)kb * kBK : 0u;
    const __amdgpu_buffer_rsrc_t ra = live ? a_rsrc : null_rsrc;
    const __amdgpu_buffer_rsrc_t rb = live ? b_rsrc : null_rsrc;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) dma16(ra, a_off[i], koff, S.a + (i * kWaves + wave) * 1024);
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) dma16(rb, b_off[i], koff, S.b + (i * kWaves + wave) * 1024);
  };

  // scales: rows wm*64 + i*32 + lane % 32; the wave's 128 columns are one B block
  const int g = lane >> 5;
  const int lr = lane & 31;
  const __amdgpu_buffer_rsrc_t sa_rsrc = make_rsrc(p.sa + row_base * p.sa_ms, 0xFFFFFFFFu);
  uint32_t sa_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wm * 64 + i * 32 + lr;
    sa_off[i] = (uint32_t)((r < rows_valid ? r : rows_valid - 1) * p.sa_ms * 4);
  }
  const __amdgpu_buffer_rsrc_t sb_rsrc = make_rsrc(SB + ((n0 + wn * 128) >> 7) * p.sb_ns, 0xFFFFFFFFu);
  struct ScaleRegs {
    float sa[2];
    float sb;
  };
  auto load_scales = [&](int kb, ScaleRegs& s) {
    const bool live = kb < nkb;
    const __amdgpu_buffer_rsrc_t ra = live ? sa_rsrc : null_rsrc;
    const uint32_t ka = live ? (uint32_t)(kb * p.sa_ks * 4) : 0u;
    const uint32_t kbo = live ? (uint32_t)(kb * p.sb_ks * 4) : 0u;
#pragma unroll
    for (int i = 0; i < 2; ++i) s.sa[i] = load_f32(ra, sa_off[i], ka);
    s.sb = load_f32(live ? sb_rsrc : null_rsrc, 0u, kbo);
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // The accumulator holds D / u[i], one unit per lane and row tile i: the
  // leftover factor f of the last group (1 at the start, and throughout for
  // power-of-two scales).  A group's split gives the instruction's E8M0
  // bytes and r = u / f, the rescale that brings the accumulator to the
  // group's units before its products are chained in (none when f = u).
  // Scales are positive (an E8M0 scale has no zero), so f > 0.  The splits
  // run two groups ahead; those of the groups past the end of K (whose
  // scale loads read nothing) leave u as it is.
  float u[2] = {1.f, 1.f};
  struct Split {
    int ea[2], eb;
    float r[2];
    bool rescale;  // some r of the wave differs from 1
  };
  auto split = [&](const ScaleRegs& sr, int kb) {
    Split sp;
    bool resc = false;
    const bool live = kb < nkb;
    const float sb = sr.sb;
    sp.eb = (int)((__float_as_uint(sb) >> 23) & 0xFFu);
    const float fb = __builtin_amdgcn_ldexpf(sb, 127 - sp.eb);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sp.ea[i] = (int)((__float_as_uint(sr.sa[i]) >> 23) & 0xFFu);
      const float f = __builtin_amdgcn_ldexpf(sr.sa[i], 127 - sp.ea[i]) * fb;
      // u / f, exactly 1 when f = u (a reciprocal refined by one Newton step
      // otherwise; its last-bit error is far below the FP8 MFMA's)
      float rf = __builtin_amdgcn_rcpf(f);
      rf = __builtin_fmaf(__builtin_fmaf(-f, rf, 1.0f), rf, rf);
      sp.r[i] = f == u[i] ? 1.0f : u[i] * rf;
      u[i] = live ? f : u[i];
      resc = resc || sp.r[i] != 1.f;
    }
    sp.rescale = __builtin_amdgcn_ballot_w64(resc) != 0;
    return sp;
  };

  // LDS fragment offsets: rows wm*64 + i*32 + lr (A) and wn*128 + j*32 + lr
  // (B) all have swz(row) = swz(lr); lane half g reads chunks 4s + 2g, +1.
  const int sw = swz(lr);
  uint32_t f_off[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) f_off[s][h] = (uint32_t)(lr * 128 + (((4 * s + 2 * g + h) ^ sw) << 4));
  auto frag = [&](const uint8_t* base, uint32_t row0, int s) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row0 * 128 + f_off[s][0]);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row0 * 128 + f_off[s][1]);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  // One K group: wait for its stage, read its first slice's fragments,
  // bring the accumulator to the group's units, load the scales of group
  // kb + 2 into lsr and start the copies of group kb + 1 (scales first, so
  // that using them waits on no copy), then chain the MFMAs of its two
  // 64-byte K slices.  The stages are passed statically: with a stage picked
  // at run time the compiler cannot tell the copies' LDS target from the
  // stage being read and drains the copies before the reads.
  auto group = [&](bool units, int kb, const Stage2<4>& S, Stage2<4>& Nx, const Split& sp, ScaleRegs& lsr) {
    wait_vmcnt<0>();
    block_barrier();
    v8i af[2], bf[4];
    auto read = [&](int s) {
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = frag(S.a, wm * 64 + i * 32, s);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = frag(S.b, wn * 128 + j * 32, s);
    };
    auto mfmas = [&]() {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af[i], acc[i][j], 0, 0, 0, sp.eb, 0,
                                                                       sp.ea[i]);
      __builtin_amdgcn_sched_barrier(0);  // one slice's fragments live at a time
    };
    read(0);  // in flight during the rescale
    if (units && sp.rescale) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= sp.r[i];
    }
    // issued here, in the block of the first MFMAs, so that they interleave
    load_scales(kb + 2, lsr);
    issue(kb + 1, Nx);
    mfmas();
    read(1);
    mfmas();
  };

  ScaleRegs sr0{}, sr1{};
  load_scales(0, sr0);
  load_scales(1, sr1);
  issue(0, stage0);
  Split sp0 = split(sr0, 0);
  Split sp1 = split(sr1, 1);
  // Pairs of groups with nothing to rescale (power-of-two scales) run in a
  // loop without the rescale code: its branch, even untaken, splits the
  // group's block and costs about 6% here.  From the first pair with a
  // rescale on, the wave runs the other loop to the end of K; every wave
  // meets one barrier per group on either path.
  int kb = 0;
  for (; kb + 2 <= nkb && !sp0.rescale && !sp1.rescale; kb += 2) {
    group(false, kb, stage0, stage1, sp0, sr0);
    group(false, kb + 1, stage1, stage0, sp1, sr1);
    sp0 = split(sr0, kb + 2);
    sp1 = split(sr1, kb + 3);
  }
  for (; kb + 2 <= nkb; kb += 2) {
    group(true, kb, stage0, stage1, sp0, sr0);
    group(true, kb + 1, stage1, stage0, sp1, sr1);
    sp0 = split(sr0, kb + 2);
    sp1 = split(sr1, kb + 3);
  }
  if (kb < nkb) group(true, kb, stage0, stage1, sp0, sr0);
  wait_vmcnt<0>();

  // epilogue: lane holds row lr of row tile i, columns 8q + 4g .. +3 of
  // column tile j; D = acc * u
  if constexpr (CT == 0) {
    const bool vec = p.vec_store != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + i * 32 + lr;
      if (row >= rows_valid) continue;
      const int64_t grow = row_base + row;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = n0 + wn * 128 + j * 32 + 8 * q + 4 * g;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * q + t] * u[i];
          store_c4<CT>(p.c, grow * p.ldc + col, v, vec);
        }
    }
  } else {
    // FP32 output: one copy of the stores per width, so that the aligned
    // copy keeps its 16-byte stores (with a per-store choice the compiler
    // merges the two forms into narrower ones).
    auto epilogue = [&](auto vec_c) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + lr;
        if (row >= rows_valid) continue;
        const int64_t grow = row_base + row;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t col = n0 + wn * 128 + j * 32 + 8 * q + 4 * g;
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * q + t] * u[i];
            store_c4<CT>(p.c, grow * p.ldc + col, v, decltype(vec_c)::value);
          }
      }
    };
    if (p.vec_store != 0)
      epilogue(BoolTag<true>{});
    else
      epilogue(BoolTag<false>{});
  }
}

template <int CT, bool GROUPED>
hipError_t launch_mx(const KParams& kp, hipStream_t st) {
  hipLaunchKernelGGL((gemm_mx_kernel<CT, GROUPED>), dim3(kp.nblocks), dim3(kThreads), 0, st, kp);
  return hipGetLastError();
}

template <int CT, bool GROUPED, int JT>
hipError_t launch_rescale(const KParams& kp, hipStream_t st) {
  if constexpr (GROUPED)
    hipLaunchKernelGGL((gemm_rescale_grouped_kernel<CT, JT>), dim3(kp.nblocks), dim3(kThreads), 0, st, kp);
  else
    hipLaunchKernelGGL((gemm_rescale_kernel<CT, JT>), dim3(kp.nblocks), dim3(kThreads), 0, st, kp);
  return hipGetLastError();
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
    case kModeFp8Mx: return launch_grouped_or_dense<CT, BMODE, kModeFp8Mx>(kp, grouped, st);
    default: return launch_grouped_or_dense<CT, BMODE, kModeFp8NoPromo>(kp, grouped, st);
  }
}

}  // namespace

ColumnPlan plan_columns(int64_t tiles_m, int64_t N, int cus) {
  // Column tiles of 256 and 192 with 256 n256 + 192 n192 = N; the split
  // with the fewest CU rounds (a 192-column tile costs 3/4 of a 256-column
  // one) wins, ties going to more 256-column tiles.  cus <= 0: 256-column
  // tiles only.
  ColumnPlan best{0, 0};
  if (N % 64 != 0 || N == 0) return best;
  if (cus <= 0) {
    if (N % 256 == 0) best.n256 = N / 256;
    return best;
  }
  int64_t best_cost = -1;  // in quarter rounds
  for (int64_t n256 = N / 256; n256 >= 0; --n256) {
    const int64_t rem = N - 256 * n256;
    if (rem % 192 != 0) continue;
    const int64_t n192 = rem / 192;
    const int64_t r256 = (tiles_m * n256 + cus - 1) / cus;
    const int64_t r192 = (tiles_m * n192 + cus - 1) / cus;
    const int64_t cost = 4 * r256 + 3 * r192;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = ColumnPlan{n256, n192};
    }
  }
  return best;
}

GemmPlan plan_gemm(const GemmArgs& g, int cus) {
  GemmPlan pl{};
  pl.kernel = GemmKernel::kNone;
  pl.mode = (g.flags & FP8FG_GEMM_NO_PROMOTION)  ? kModeFp8NoPromo
            : (g.flags & FP8FG_GEMM_E8M0_SCALES) ? kModeFp8Mx
            : (g.flags & FP8FG_GEMM_FP8_MFMA)    ? kModeFp8
                                                 : kModeExact;
  const bool grouped = g.G > 0;
  const int64_t tiles_m = grouped ? (g.M + kBM - 1) / kBM + g.G : (g.M + kBM - 1) / kBM;
  if (g.M == 0 || g.N == 0 || tiles_m == 0) return pl;
  const bool block = g.b_scale_mode == FP8FG_BSCALE_BLOCK128;
  // E8M0 scales with block scales and N % 256 == 0: 256 x 256 tiles.
  if (pl.mode == kModeFp8Mx && block && g.N % 256 == 0) {
    pl.kernel = GemmKernel::kMx;
    pl.threads = kThreads;
    pl.launch[0] = GemmLaunch{g.N / 256, 0, tiles_m * (g.N / 256)};
    return pl;
  }
  // Exact path with block scales: the weight-streaming kernel on 64x128
  // tiles, two workgroups per CU, for few rows per expert, a dense M of at
  // most one 64-row tile, or a dense grid of 256x256 tiles that would fill
  // at most half of the CUs (small M x N with a long K: per CU the 64x128
  // tiles deliver about half the rate of the 256x256 ones, so they win once
  // they keep at least twice the CUs busy).  Both tile shapes give every
  // output element bit for bit the same value; the flags
  // FP8FG_GEMM_TILES_WIDE / _NARROW fix the choice.
  const int64_t wide_tiles = tiles_m * ((g.N + 255) / 256);
  const bool narrow = (g.flags & FP8FG_GEMM_TILES_NARROW) ? true
                      : (g.flags & FP8FG_GEMM_TILES_WIDE) ? false
                      : grouped ? g.M <= kStreamRowsPerExpert * g.G
                                : (g.M <= kWBM || wide_tiles * 2 <= cus);
  if (pl.mode == kModeExact && block && narrow) {
    const int64_t tm = grouped ? (g.M + kWBM - 1) / kWBM + g.G : (g.M + kWBM - 1) / kWBM;
    const int64_t tn = g.N / (32 * kStreamWaves);
    pl.kernel = GemmKernel::kStream;
    pl.threads = 64 * kStreamWaves;
    pl.launch[0] = GemmLaunch{tn, 0, tm * tn};
    return pl;
  }
  // The default path with block scales runs the rescaled-accumulation
  // kernel on 256-column tiles and possibly a second launch of 192-column
  // tiles, the split that fills the CUs best (for a grouped GEMM tiles_m
  // counts the row tiles of the worst case, and 7 more workgroups let the
  // kernel start its 128-row tiles at a multiple of 8).  Both tile widths
  // compute every output element with the same operations in the same
  // order.
  if (pl.mode == kModeExact && block) {
    const ColumnPlan cp = plan_columns(tiles_m, g.N, cus);
    const int64_t spare = grouped ? 7 : 0;
    if (cp.n256 + cp.n192 > 0) {
      pl.kernel = GemmKernel::kRescale;
      pl.threads = kThreads;
      if (cp.n256 > 0) pl.launch[0] = GemmLaunch{cp.n256, 0, tiles_m * cp.n256 + spare};
      if (cp.n192 > 0) pl.launch[1] = GemmLaunch{cp.n192, 256 * cp.n256, tiles_m * cp.n192 + spare};
      return pl;
    }
  }
  pl.kernel = GemmKernel::kBlockscaled;
  pl.threads = kThreads;
  pl.launch[0] = GemmLaunch{g.N / kBN, 0, tiles_m * (g.N / kBN)};
  return pl;
}

hipError_t launch_gemm(const GemmArgs& g, const GemmPlan& pl, hipStream_t st) {
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
  const int esize = g.c_type == 0 ? 2 : 4;
  kp.vec_store = (reinterpret_cast<uintptr_t>(g.c) % (4 * esize) == 0) && (g.ldc % 4 == 0);
  const bool grouped = g.G > 0;
  const bool bf = g.c_type == 0;
  hipError_t e = hipSuccess;
  for (int l = 0; l < 2 && e == hipSuccess; ++l) {
    const GemmLaunch& L = pl.launch[l];
    if (L.nblocks <= 0) continue;
    kp.tiles_n = (int)L.tiles_n;
    kp.n_base = L.n_base;
    kp.nblocks = (int)L.nblocks;
    switch (pl.kernel) {
      case GemmKernel::kMx:
        e = bf ? (grouped ? launch_mx<0, true>(kp, st) : launch_mx<0, false>(kp, st))
               : (grouped ? launch_mx<1, true>(kp, st) : launch_mx<1, false>(kp, st));
        break;
      case GemmKernel::kStream:
        e = bf ? (grouped ? launch_stream<0, true>(kp, st) : launch_stream<0, false>(kp, st))
               : (grouped ? launch_stream<1, true>(kp, st) : launch_stream<1, false>(kp, st));
        break;
      case GemmKernel::kRescale:
        if (l == 0)
          e = bf ? (grouped ? launch_rescale<0, true, 4>(kp, st) : launch_rescale<0, false, 4>(kp, st))
                 : (grouped ? launch_rescale<1, true, 4>(kp, st) : launch_rescale<1, false, 4>(kp, st));
        else
          e = bf ? (grouped ? launch_rescale<0, true, 3>(kp, st) : launch_rescale<0, false, 3>(kp, st))
                 : (grouped ? launch_rescale<1, true, 3>(kp, st) : launch_rescale<1, false, 3>(kp, st));
        break;
      case GemmKernel::kBlockscaled:
        if (bf)
          e = g.b_scale_mode == 0 ? launch_mode<0, 0>(kp, pl.mode, grouped, st)
                                  : launch_mode<0, 1>(kp, pl.mode, grouped, st);
        else
          e = g.b_scale_mode == 0 ? launch_mode<1, 0>(kp, pl.mode, grouped, st)
                                  : launch_mode<1, 1>(kp, pl.mode, grouped, st);
        break;
      case GemmKernel::kNone:
        break;
    }
  }
  return e;
}

}  // namespace fp8fg
