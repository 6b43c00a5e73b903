// Fine-grained FP8 quantizers for gfx950.
//
// The method ([why-be] and [thedaegu] paragraphs on fine-grained
// quantization; page keys in include/fp8fg.h): the max-abs of every 1x128
// activation tile or 128x128 weight block is computed online, a scale is
// derived so that it lands on the largest E4M3 value, and the tile is
// quantized to E4M3.  In the backward pass activations are re-tiled from
// 1x128 to 128x1 ([why-be], backward-pass paragraph), and some activations
// use power-of-two scales.
//
// Both kernels are HBM-streaming: each input element is read once and each
// output byte written once, with non-temporal loads and stores (nothing is
// reused; streaming past the caches measured 5-12% faster than ordinary
// accesses on the 4096 x 7168 activations).
//
// quant_1x128: 16 lanes own one tile (8 consecutive elements per lane, one
//   16-byte load for bf16), so a wave reads 4 consecutive tiles = 1 KiB of
//   contiguous bf16.  The tile max is a 4-step DPP reduction inside a DPP
//   row.  Each lane packs its 8 bytes with two v_cvt_pk_fp8_f32 pairs and
//   writes them with one 8-byte store.  A grid-stride loop keeps 2 tiles per
//   lane-group in flight; the tile -> (row, tile column) split is a 32-bit
//   multiply-high division.
//
// quant_tile128: one 256-thread workgroup per 128x128 block.  Thread
//   (rg, cg) = (tid / 16, tid % 16) holds rows 8rg..8rg+7 x columns
//   8cg..8cg+7 in registers, undecoded; a row of the block is read by 16
//   consecutive lanes (fully used 256-byte segments for bf16).  Column (128x1) or block
//   maxima are reduced through LDS.  For the transposed layouts the bytes
//   are converted directly in column order -- the conversion instruction
//   takes any two registers -- and staged through LDS, so that each lane
//   stores 16 contiguous bytes and a wave writes 8 whole 128-byte output rows;
//   the staging buffer reuses the LDS of the column-max partials.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "device_common.h"
#include "launch.h"

namespace fp8fg {

namespace {

constexpr int kQThreads = 256;
constexpr int kGroupsPerBlock = kQThreads / 16;
constexpr int kUnroll = 2;
constexpr int kTPitch = 144;  // LDS row pitch (bytes) of the transposing store
// 1x128 grid: up to 28 workgroups of 256 threads per CU (for the 4096 x 7168
// activations exactly one pass of two tiles per lane group); 14 measured 10%
// slower
constexpr int k1x128BlocksPerCu = 28;

// n / d for 32-bit n by multiply-high and shift (Granlund & Montgomery,
// "Division by invariant integers using multiplication", PLDI 1994):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (umulhi(n, m) + n) >> l for every n < 2^32 (the sum is formed in
// 64 bits).
struct FastDiv {
  uint32_t d, m, l;
};

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  const uint64_t t = (uint64_t)__umulhi(n, f.m) + n;
  return (uint32_t)(t >> f.l);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Non-temporal 16- and 8-byte accesses.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ void st_nt8(void* p, uint2 v) {
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

template <int XT>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t off, float v[8]) {
  if constexpr (XT == 0) {
    const uint4 w = ld_nt16(reinterpret_cast<const uint16_t*>(x) + off);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
    const float* p = reinterpret_cast<const float*>(x) + off;
    const uint4 a = ld_nt16(p), b = ld_nt16(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

// Lane group g of the grid handles tiles g, g + G, ... (G = number of lane
// groups), two per iteration so that both loads are in flight before either
// is processed.  ORDER 0 numbers the tiles row-major (t = r * tiles_per_row
// + tc): a wave's four tiles lie side by side in one row, and with
// row-major scales (s_ts = 1) their four scales are one 16-byte store.
// ORDER 1, for scales stored group-major (s_rs = 1), numbers them in bands
// of 16 rows, tile column by tile column (t = 16 tpr band + 16 tc + r % 16):
// a wave's four tiles are four consecutive rows of one tile column, whose
// scales are adjacent; the last band may have fewer rows.  (Scattered
// 4-byte scale stores cost 20% more written bytes than the output itself.)
template <int ORDER>
__device__ __forceinline__ void tile_rc(uint32_t t, const FastDiv& tpr, const FastDiv& band,
                                        uint32_t rows, uint32_t& r, uint32_t& tc) {
  if constexpr (ORDER == 0) {
    r = fast_div(t, tpr);
    tc = t - r * tpr.d;
  } else {
    const uint32_t b = fast_div(t, band);
    const uint32_t u = t - b * band.d;
    const uint32_t h = rows - 16u * b;  // rows in this band (16 except in the last)
    if (h >= 16u) {
      tc = u >> 4;
      r = 16u * b + (u & 15u);
    } else {
      tc = u / h;
      r = 16u * b + (u - tc * h);
    }
  }
}

template <int XT, int RULE, int ORDER>
__global__ __launch_bounds__(kQThreads) void quant_1x128_kernel(
    const void* __restrict__ x, uint32_t ntiles, FastDiv tpr, FastDiv band, uint32_t rows,
    int64_t ldx, uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t s_rs,
    int64_t s_ts) {
  const int lane16 = threadIdx.x & 15;
  const uint32_t group = blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const uint32_t ngroups = gridDim.x * kGroupsPerBlock;

  for (uint32_t t0 = group; t0 < ntiles; t0 += kUnroll * ngroups) {
    float v[kUnroll][8];
    uint32_t r[kUnroll], tc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t t = t0 + u * ngroups;
      if (t < ntiles) {
        tile_rc<ORDER>(t, tpr, band, rows, r[u], tc[u]);
        load8<XT>(x, (int64_t)r[u] * ldx + tc[u] * 128 + lane16 * 8, v[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t0 + u * ngroups >= ntiles) continue;
      float m = fabsf(v[u][0]);
#pragma unroll
      for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(v[u][i]));
      m = row16_max(m);
      const TileScale sc = RULE == 0 ? scale_amax(m) : scale_pow2(m);
      float qv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = v[u][i];
      quotient8<RULE>(qv, sc);
      uint2 out;
      out.x = pack4_e4m3(qv[0], qv[1], qv[2], qv[3]);
      out.y = pack4_e4m3(qv[4], qv[5], qv[6], qv[7]);
      st_nt8(q + (int64_t)r[u] * ldq + tc[u] * 128 + lane16 * 8, out);
      if (lane16 == 0) s[(int64_t)r[u] * s_rs + (int64_t)tc[u] * s_ts] = sc.s;
    }
  }
}

// ---------------------------------------------------------------- 128 x 128
// A thread's 8 x 8 elements stay in registers in their input encoding (bf16
// pairs, f32, or E4M3 bytes) and are decoded where they are used: once for
// the maxima and once for the quotients.  That keeps the kernel at 8
// workgroups per CU (at most 64 VGPRs), where holding 64 decoded floats
// allowed 5-6; the requantizer's 1792-block grid then fits in one round on
// 256 CUs.  An f32 input is its own decoded form (64 VGPRs of raw data), so
// that instantiation keeps the compiler's default register budget.
template <int XT>
struct RawRow;
template <>
struct RawRow<0> {  // 8 bf16
  uint4 w;
};
template <>
struct RawRow<1> {  // 8 f32
  uint4 a, b;
};
template <>
struct RawRow<2> {  // 8 E4M3 bytes
  uint2 w;
};

template <int XT>
__device__ __forceinline__ RawRow<XT> load_raw(const void* __restrict__ x, int64_t off) {
  RawRow<XT> r;
  if constexpr (XT == 0) {
    r.w = ld_nt16(reinterpret_cast<const uint16_t*>(x) + off);
  } else if constexpr (XT == 1) {
    const float* p = reinterpret_cast<const float*>(x) + off;
    r.a = ld_nt16(p);
    r.b = ld_nt16(p + 4);
  } else {
    r.w = ld_nt8(reinterpret_cast<const uint8_t*>(x) + off);
  }
  return r;
}

// Elements J and J + 1 (J even) of a raw row, exactly as fp32.
template <int J, int XT>
__device__ __forceinline__ void raw_pair(const RawRow<XT>& r, float& a, float& b) {
  static_assert(J % 2 == 0 && J < 8, "pairs start at even columns");
  if constexpr (XT == 0) {
    const uint32_t w = J == 0 ? r.w.x : J == 2 ? r.w.y : J == 4 ? r.w.z : r.w.w;
    a = bf16_lo(w);
    b = bf16_hi(w);
  } else if constexpr (XT == 1) {
    const uint4& h = J < 4 ? r.a : r.b;
    a = __uint_as_float((J & 3) == 0 ? h.x : h.z);
    b = __uint_as_float((J & 3) == 0 ? h.y : h.w);
  } else {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)(J < 4 ? r.w.x : r.w.y), (J & 2) != 0);
    a = f[0];
    b = f[1];
  }
}

// Hides a raw row's registers from the optimizer (no instruction is
// emitted): the values decoded before this point cannot be reused after it,
// so the second pass decodes again instead of keeping 64 floats live.
template <int XT>
__device__ __forceinline__ void refresh(RawRow<XT>& r) {
  if constexpr (XT == 0) {
    asm volatile("" : "+v"(r.w.x), "+v"(r.w.y), "+v"(r.w.z), "+v"(r.w.w));
  } else if constexpr (XT == 1) {
    asm volatile("" : "+v"(r.a.x), "+v"(r.a.y), "+v"(r.a.z), "+v"(r.a.w));
    asm volatile("" : "+v"(r.b.x), "+v"(r.b.y), "+v"(r.b.z), "+v"(r.b.w));
  } else {
    asm volatile("" : "+v"(r.w.x), "+v"(r.w.y));
  }
}

template <int J>
struct ColTag {
  static constexpr int value = J;
};
template <typename F, int... P>
__device__ __forceinline__ void for_pairs_impl(F&& f, std::integer_sequence<int, P...>) {
  (f(ColTag<2 * P>{}), ...);
}
// f(ColTag<0>{}), f(ColTag<2>{}), .. f(ColTag<6>{}): the first column of
// each pair as a compile-time constant.
template <typename F>
__device__ __forceinline__ void for_pairs(F&& f) {
  for_pairs_impl(f, std::make_integer_sequence<int, 4>{});
}

template <int XT, int RULE, bool PER_COLUMN, bool TRANSPOSE>
__global__ __launch_bounds__(kQThreads, XT == 1 ? 1 : 8) void quant_tile128_kernel(
    const void* __restrict__ x, int64_t ldx, const float* __restrict__ xs, int64_t xs_rs,
    int64_t xs_ts, uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t s_a,
    int64_t s_b) {
  static_assert(!PER_COLUMN || TRANSPOSE, "128x1 tiles are written transposed");
  // The transposed store is staged in LDS; the column-max partials (16 x 128
  // floats) use the first 8 KB of that buffer before it is written (two
  // barriers separate their last read from the first staging write).
  __shared__ __align__(16) uint8_t tbuf[TRANSPOSE ? 128 * kTPitch : 16];
  __shared__ TileScale col_sc[PER_COLUMN ? 128 : 1];
  __shared__ uint32_t blk_max;
  float (*part)[128] = reinterpret_cast<float (*)[128]>(tbuf);

  const int tid = threadIdx.x;
  const int cg = tid & 15;
  const int rg = tid >> 4;
  const int64_t r0 = (int64_t)blockIdx.y * 128;
  const int64_t c0 = (int64_t)blockIdx.x * 128;

  if (!PER_COLUMN && tid == 0) blk_max = 0u;

  RawRow<XT> raw[8];
  float rsc[8];  // requantization: the input scale of each row
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = r0 + rg * 8 + i;
    raw[i] = load_raw<XT>(x, row * ldx + c0 + cg * 8);
    if constexpr (XT == 2) rsc[i] = xs[row * xs_rs + (c0 >> 7) * xs_ts];
  }
  // elements (i, J) and (i, J + 1) of the thread's block; for
  // requantization RN32(dec(q1) * s1)
  auto pair = [&](int i, auto col, float& a, float& b) {
    raw_pair<decltype(col)::value>(raw[i], a, b);
    if constexpr (XT == 2) {
      a *= rsc[i];
      b *= rsc[i];
    }
  };

  TileScale bsc{};  // the block's scale (128x128 tiles)
  if constexpr (PER_COLUMN) {
    for_pairs([&](auto col) {
      float ma = 0.0f, mb = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        float a0, b0, a1, b1;
        pair(i, col, a0, b0);
        pair(i + 1, col, a1, b1);
        ma = fmaxf(fmaxf(ma, fabsf(a0)), fabsf(a1));  // one three-input max
        mb = fmaxf(fmaxf(mb, fabsf(b0)), fabsf(b1));
      }
      part[rg][cg * 8 + decltype(col)::value] = ma;
      part[rg][cg * 8 + decltype(col)::value + 1] = mb;
    });
    __syncthreads();
    if (tid < 128) {
      float m = part[0][tid];
#pragma unroll
      for (int g = 1; g < 16; ++g) m = fmaxf(m, part[g][tid]);
      const TileScale sc = RULE == 0 ? scale_amax(m) : scale_pow2(m);
      col_sc[tid] = sc;
      s[(c0 + tid) * s_a + (r0 >> 7) * s_b] = sc.s;
    }
    __syncthreads();
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      for_pairs([&](auto col) {
        float a, b;
        pair(i, col, a, b);
        m = fmaxf(fmaxf(m, fabsf(a)), fabsf(b));  // one three-input max
      });
    m = row16_max(m);
    __syncthreads();  // blk_max initialised
    if ((tid & 15) == 0) atomicMax(&blk_max, __float_as_uint(m));  // m >= 0: integer order == float order
    __syncthreads();
    bsc = RULE == 0 ? scale_amax(__uint_as_float(blk_max)) : scale_pow2(__uint_as_float(blk_max));
    if (tid == 0) s[(r0 >> 7) * s_a + (c0 >> 7) * s_b] = bsc.s;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) refresh(raw[i]);

  if constexpr (TRANSPOSE) {
    // Output row c (an input column) is 128 contiguous bytes.  Stage the
    // block through LDS so that every lane stores 16 bytes and a wave writes
    // 8 whole rows: row pitch 144 bytes and 16-byte chunks XOR-swizzled by
    // (c / 16) % 8 keep the scattered 8-byte writes and the row reads off
    // the same LDS banks.  The bytes are formed a pair of columns at a
    // time: the conversion instruction takes any two registers.
    for_pairs([&](auto col) {
      constexpr int J = decltype(col)::value;
      float va[8], vb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pair(i, col, va[i], vb[i]);
      TileScale ca = bsc, cb = bsc;
      if constexpr (PER_COLUMN) {
        ca = col_sc[cg * 8 + J];
        cb = col_sc[cg * 8 + J + 1];
      }
      quotient8<RULE>(va, ca);
      quotient8<RULE>(vb, cb);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float* v = h ? vb : va;
        const int c = cg * 8 + J + h;
        uint2 out;
        out.x = pack4_e4m3(v[0], v[1], v[2], v[3]);
        out.y = pack4_e4m3(v[4], v[5], v[6], v[7]);
        const int chunk = (rg >> 1) ^ ((c >> 4) & 7);
        *reinterpret_cast<uint2*>(tbuf + c * kTPitch + chunk * 16 + (rg & 1) * 8) = out;
      }
    });
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int k = it * kQThreads + tid;
      const int c = k >> 3;
      const int chunk = k & 7;
      const uint4 w = *reinterpret_cast<const uint4*>(tbuf + c * kTPitch + ((chunk ^ ((c >> 4) & 7)) << 4));
      st_nt16(q + (c0 + c) * ldq + r0 + chunk * 16, w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      for_pairs([&](auto col) { pair(i, col, v[decltype(col)::value], v[decltype(col)::value + 1]); });
      quotient8<RULE>(v, bsc);
      uint2 out;
      out.x = pack4_e4m3(v[0], v[1], v[2], v[3]);
      out.y = pack4_e4m3(v[4], v[5], v[6], v[7]);
      st_nt8(q + (r0 + rg * 8 + i) * ldq + c0 + cg * 8, out);
    }
  }
}

FastDiv make_fast_div(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

template <int XT, int RULE>
hipError_t launch_1x128_t(const RowtileArgs& a, hipStream_t st) {
  const int64_t tpr = a.cols / 128;
  const int64_t ntiles = a.rows * tpr;
  const int64_t per_block = kGroupsPerBlock * kUnroll;
  const int64_t want = (ntiles + per_block - 1) / per_block;
  const int64_t cap = (int64_t)device_cu_count() * k1x128BlocksPerCu;
  const int64_t blocks = want < cap ? want : cap;
  const FastDiv fd_tpr = make_fast_div((uint32_t)tpr);
  const FastDiv fd_band = make_fast_div((uint32_t)(16 * tpr));
  // (the band order needs 16 * tiles_per_row < 2^32)
  if (a.s_rs == 1 && tpr < ((int64_t)1 << 28)) {
    hipLaunchKernelGGL((quant_1x128_kernel<XT, RULE, 1>), dim3((unsigned)blocks), dim3(kQThreads), 0, st,
                       a.x, (uint32_t)ntiles, fd_tpr, fd_band, (uint32_t)a.rows, a.ldx, a.q, a.ldq, a.s,
                       a.s_rs, a.s_ts);
  } else {
    hipLaunchKernelGGL((quant_1x128_kernel<XT, RULE, 0>), dim3((unsigned)blocks), dim3(kQThreads), 0, st,
                       a.x, (uint32_t)ntiles, fd_tpr, fd_band, (uint32_t)a.rows, a.ldx, a.q, a.ldq, a.s,
                       a.s_rs, a.s_ts);
  }
  return hipGetLastError();
}

template <int XT, int RULE, bool PC, bool TR>
hipError_t launch_t128_t(const Tile128Args& a, hipStream_t st) {
  dim3 grid((unsigned)(a.cols / 128), (unsigned)(a.rows / 128));
  hipLaunchKernelGGL((quant_tile128_kernel<XT, RULE, PC, TR>), grid, dim3(kQThreads), 0, st, a.x,
                     a.ldx, a.xs, a.xs_rs, a.xs_ts, a.q, a.ldq, a.s, a.s_a, a.s_b);
  return hipGetLastError();
}

template <int XT, int RULE>
hipError_t dispatch_t128_layout(const Tile128Args& a, hipStream_t st) {
  // 128x1 tiles are always written transposed (the ABI offers no other form)
  if (a.per_column) return launch_t128_t<XT, RULE, true, true>(a, st);
  return a.transpose ? launch_t128_t<XT, RULE, false, true>(a, st)
                     : launch_t128_t<XT, RULE, false, false>(a, st);
}

}  // namespace

hipError_t launch_quant_1x128(const RowtileArgs& a, hipStream_t st) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  if (a.x_type == 0) return a.rule == 0 ? launch_1x128_t<0, 0>(a, st) : launch_1x128_t<0, 1>(a, st);
  return a.rule == 0 ? launch_1x128_t<1, 0>(a, st) : launch_1x128_t<1, 1>(a, st);
}

hipError_t launch_quant_tile128(const Tile128Args& a, hipStream_t st) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  switch (a.x_type) {
    case 0:
      return a.rule == 0 ? dispatch_t128_layout<0, 0>(a, st) : dispatch_t128_layout<0, 1>(a, st);
    case 1:
      return a.rule == 0 ? dispatch_t128_layout<1, 0>(a, st) : dispatch_t128_layout<1, 1>(a, st);
    default:  // e4m3 requantization: 128x1 tiles, transposed output only
      return a.rule == 0 ? launch_t128_t<2, 0, true, true>(a, st)
                         : launch_t128_t<2, 1, true, true>(a, st);
  }
}

}  // namespace fp8fg
