// Device helpers shared by the quantizer and GEMM kernels (gfx950 only).
//
// FP8 here is OCP E4M3 (bias 7, largest finite 448), which gfx950's
// conversion and matrix instructions use natively.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8fg {

constexpr float kE4M3Max = 448.0f;
constexpr float kFltMinNormal = 1.17549435082228750797e-38f;  // 2^-126

// bf16 halves of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// DPP row controls (a DPP row is 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over the 16 lanes of a DPP row; every lane of the row gets the result.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppRowMirror>(v));
  return v;
}

// A tile's scale s (dequantization multiplier) and y = RN(1/s).
struct TileScale {
  float s;
  float y;
};

// s = max(RN(amax / 448), 2^-126); y = RN(1 / s).  Both divisions are the
// compiler's correctly rounded fp32 division (no fast-math is used).
__device__ __forceinline__ TileScale scale_amax(float amax) {
  float s = fmaxf(amax / kE4M3Max, kFltMinNormal);
  return {s, 1.0f / s};
}

// s = max(2^k, 2^-126) with k the least integer such that 448 * 2^k >= amax.
// With amax = 1.f * 2^e: amax / 448 = (1.f / 1.75) * 2^(e - 8), so
// k = e - 8 when 1.f <= 1.75 (mantissa field <= 0x600000) and e - 7 otherwise.
// Zero and subnormal amax fall below the floor.
__device__ __forceinline__ TileScale scale_pow2(float amax) {
  const uint32_t u = __float_as_uint(amax);
  int k = (int)((u >> 23) & 0xFFu) - 127 - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  k = k < -126 ? -126 : k;
  return {__uint_as_float((uint32_t)(k + 127) << 23), __uint_as_float((uint32_t)(127 - k) << 23)};
}

// Correctly rounded x / s from y = RN(1/s) (Markstein's FMA-based quotient
// correction; P. Markstein, IBM J. Res. Dev. 34(1), 1990).  The residual is
// formed as s*q0 - x so that x = -0 keeps its sign.
__device__ __forceinline__ float div_by_scale(float x, float s, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(s, q0, -x);
  return __builtin_fmaf(-r, y, q0);
}

// Four fp32 values -> four E4M3 bytes (first value in the lowest byte),
// round-to-nearest-even; values are clamped to +-448 first (saturation).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Four E4M3 bytes of a word -> fp32 (exact).
__device__ __forceinline__ void unpack4_e4m3(uint32_t w, float out[4]) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

}  // namespace fp8fg
