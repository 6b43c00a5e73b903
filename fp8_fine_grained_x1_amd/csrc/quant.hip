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
// output byte written once.
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
//   8cg..8cg+7 in registers; a row of the block is read by 16 consecutive
//   lanes (fully used 256-byte segments for bf16).  Column (128x1) or block
//   maxima are reduced through LDS.  For the transposed layouts the bytes
//   are converted directly in column order -- the conversion instruction
//   takes any two registers -- and staged through LDS, so that each lane
//   stores 16 contiguous bytes and a wave writes 8 whole 128-byte output rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace fp8fg {

namespace {

constexpr int kQThreads = 256;
constexpr int kGroupsPerBlock = kQThreads / 16;
constexpr int kUnroll = 2;
constexpr int kTPitch = 144;  // LDS row pitch (bytes) of the transposing store

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

template <int XT>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t off, float v[8]) {
  if constexpr (XT == 0) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Tiles are numbered row-major (t = r * tiles_per_row + tc); lane group g of
// the grid handles tiles g, g + G, ... (G = number of lane groups), two per
// iteration so that both loads are in flight before either is processed.
template <int XT, int RULE>
__global__ __launch_bounds__(kQThreads) void quant_1x128_kernel(
    const void* __restrict__ x, uint32_t ntiles, FastDiv tpr, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t s_rs, int64_t s_ts) {
  const int lane16 = threadIdx.x & 15;
  const uint32_t group = blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const uint32_t ngroups = gridDim.x * kGroupsPerBlock;

  for (uint32_t t0 = group; t0 < ntiles; t0 += kUnroll * ngroups) {
    float v[kUnroll][8];
    uint32_t r[kUnroll], tc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t t = t0 + u * ngroups;
      r[u] = fast_div(t, tpr);
      tc[u] = t - r[u] * tpr.d;
      if (t < ntiles) load8<XT>(x, (int64_t)r[u] * ldx + tc[u] * 128 + lane16 * 8, v[u]);
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
      for (int i = 0; i < 8; ++i) qv[i] = RULE == 0 ? div_by_scale(v[u][i], sc.s, sc.y) : v[u][i] * sc.y;
      uint2 out;
      out.x = pack4_e4m3(qv[0], qv[1], qv[2], qv[3]);
      out.y = pack4_e4m3(qv[4], qv[5], qv[6], qv[7]);
      *reinterpret_cast<uint2*>(q + (int64_t)r[u] * ldq + tc[u] * 128 + lane16 * 8) = out;
      if (lane16 == 0) s[(int64_t)r[u] * s_rs + (int64_t)tc[u] * s_ts] = sc.s;
    }
  }
}

// ---------------------------------------------------------------- 128 x 128
template <int XT>
__device__ __forceinline__ void load_row8(const void* __restrict__ x, int64_t off, float v[8]) {
  if constexpr (XT == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(x) + off);
    unpack4_e4m3(w.x, v);
    unpack4_e4m3(w.y, v + 4);
  } else {
    load8<XT>(x, off, v);
  }
}

template <int XT, int RULE, bool PER_COLUMN, bool TRANSPOSE>
__global__ __launch_bounds__(kQThreads) void quant_tile128_kernel(
    const void* __restrict__ x, int64_t ldx, const float* __restrict__ xs, int64_t xs_rs,
    int64_t xs_ts, uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t s_a,
    int64_t s_b) {
  __shared__ float part[16][128];
  __shared__ float col_s[128];
  __shared__ float col_y[128];
  __shared__ uint32_t blk_max;

  const int tid = threadIdx.x;
  const int cg = tid & 15;
  const int rg = tid >> 4;
  const int64_t r0 = (int64_t)blockIdx.y * 128;
  const int64_t c0 = (int64_t)blockIdx.x * 128;

  if (!PER_COLUMN && tid == 0) blk_max = 0u;

  float v[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = r0 + rg * 8 + i;
    load_row8<XT>(x, row * ldx + c0 + cg * 8, v[i]);
    if constexpr (XT == 2) {
      // requantization source: RN32(dec(q1) * s1), one input scale per row
      const float sc = xs[row * xs_rs + (c0 >> 7) * xs_ts];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = v[i][j] * sc;
    }
  }

  float ys[8], ss[8];
  if constexpr (PER_COLUMN) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float m = fabsf(v[0][j]);
#pragma unroll
      for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(v[i][j]));
      part[rg][cg * 8 + j] = m;
    }
    __syncthreads();
    if (tid < 128) {
      float m = part[0][tid];
#pragma unroll
      for (int g = 1; g < 16; ++g) m = fmaxf(m, part[g][tid]);
      const TileScale sc = RULE == 0 ? scale_amax(m) : scale_pow2(m);
      col_s[tid] = sc.s;
      col_y[tid] = sc.y;
      s[(c0 + tid) * s_a + (r0 >> 7) * s_b] = sc.s;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ss[j] = col_s[cg * 8 + j];
      ys[j] = col_y[cg * 8 + j];
    }
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[i][j]));
    m = row16_max(m);
    __syncthreads();  // blk_max initialised
    if ((tid & 15) == 0) atomicMax(&blk_max, __float_as_uint(m));  // m >= 0: integer order == float order
    __syncthreads();
    const TileScale sc = RULE == 0 ? scale_amax(__uint_as_float(blk_max)) : scale_pow2(__uint_as_float(blk_max));
    if (tid == 0) s[(r0 >> 7) * s_a + (c0 >> 7) * s_b] = sc.s;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ss[j] = sc.s;
      ys[j] = sc.y;
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[i][j] = RULE == 0 ? div_by_scale(v[i][j], ss[j], ys[j]) : v[i][j] * ys[j];

  if constexpr (TRANSPOSE) {
    // Output row c (an input column) is 128 contiguous bytes.  Stage the
    // block through LDS so that every lane stores 16 bytes and a wave writes
    // 8 whole rows: row pitch 144 bytes and 16-byte chunks XOR-swizzled by
    // (c / 16) % 8 keep the scattered 8-byte writes and the row reads off
    // the same LDS banks.
    __shared__ __align__(16) uint8_t tbuf[128 * kTPitch];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint2 out;
      out.x = pack4_e4m3(v[0][j], v[1][j], v[2][j], v[3][j]);
      out.y = pack4_e4m3(v[4][j], v[5][j], v[6][j], v[7][j]);
      const int c = cg * 8 + j;
      const int chunk = (rg >> 1) ^ ((c >> 4) & 7);
      *reinterpret_cast<uint2*>(tbuf + c * kTPitch + chunk * 16 + (rg & 1) * 8) = out;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int k = it * kQThreads + tid;
      const int c = k >> 3;
      const int chunk = k & 7;
      const uint4 w = *reinterpret_cast<const uint4*>(tbuf + c * kTPitch + ((chunk ^ ((c >> 4) & 7)) << 4));
      *reinterpret_cast<uint4*>(q + (c0 + c) * ldq + r0 + chunk * 16) = w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint2 out;
      out.x = pack4_e4m3(v[i][0], v[i][1], v[i][2], v[i][3]);
      out.y = pack4_e4m3(v[i][4], v[i][5], v[i][6], v[i][7]);
      *reinterpret_cast<uint2*>(q + (r0 + rg * 8 + i) * ldq + c0 + cg * 8) = out;
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
  const int64_t cap = (int64_t)device_cu_count() * 14;
  const int64_t blocks = want < cap ? want : cap;
  hipLaunchKernelGGL((quant_1x128_kernel<XT, RULE>), dim3((unsigned)blocks), dim3(kQThreads), 0, st,
                     a.x, (uint32_t)ntiles, make_fast_div((uint32_t)tpr), a.ldx, a.q, a.ldq, a.s,
                     a.s_rs, a.s_ts);
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
  if (a.per_column) {
    return a.transpose ? launch_t128_t<XT, RULE, true, true>(a, st)
                       : launch_t128_t<XT, RULE, true, false>(a, st);
  }
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
