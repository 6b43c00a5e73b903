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

// A tile's scale s (the stored dequantization multiplier) and what the
// quotient x / s is formed from: x * pre divided by d = s * pre, with
// y = RN(1/d).  pre is 1 unless s < 2^-64, where it is 2^64: with tiny
// scales the residual of the FMA correction below falls into FP32's
// denormal range and loses bits (the quotient of x ~ 1.4e-38 by
// s ~ 2e-36 came out one ulp low), while the same quotient of the operands
// scaled by 2^64 -- exactly, both being powers of two apart from s -- has a
// normal residual whenever x / s is large enough to matter for E4M3
// (>= 2^-11).
struct TileScale {
  float s;
  float d;
  float y;
  float pre;
};

constexpr float kTinyScale = 5.42101086242752217004e-20f;  // 2^-64
constexpr float kTinyLift = 18446744073709551616.0f;        // 2^64

// s = max(RN(amax / 448), 2^-126); the divisions are the compiler's
// correctly rounded fp32 division (no fast-math is used).
__device__ __forceinline__ TileScale scale_amax(float amax) {
  const float s = fmaxf(amax / kE4M3Max, kFltMinNormal);
  const float pre = s < kTinyScale ? kTinyLift : 1.0f;
  const float d = s * pre;
  return {s, d, 1.0f / d, pre};
}

// s = max(2^k, 2^-126) with k the least integer such that 448 * 2^k >= amax.
// With amax = 1.f * 2^e: amax / 448 = (1.f / 1.75) * 2^(e - 8), so
// k = e - 8 when 1.f <= 1.75 (mantissa field <= 0x600000) and e - 7 otherwise.
// Zero and subnormal amax fall below the floor.  x / s = x * 2^-k is exact
// (or below the E4M3 range), so y = 2^-k is all the quotient needs.
__device__ __forceinline__ TileScale scale_pow2(float amax) {
  const uint32_t u = __float_as_uint(amax);
  int k = (int)((u >> 23) & 0xFFu) - 127 - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  k = k < -126 ? -126 : k;
  const float s = __uint_as_float((uint32_t)(k + 127) << 23);
  return {s, s, __uint_as_float((uint32_t)(127 - k) << 23), 1.0f};
}

// Correctly rounded x / d from y = RN(1/d) (Markstein's FMA-based quotient
// correction; P. Markstein, IBM J. Res. Dev. 34(1), 1990), valid while the
// residual does not underflow (see TileScale).  The residual is formed as
// d*q0 - x so that x = -0 keeps its sign.
__device__ __forceinline__ float div_by_scale(float x, float d, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(d, q0, -x);
  return __builtin_fmaf(-r, y, q0);
}

// x / s under either rule (RULE 0: amax, 1: power of two).
template <int RULE>
__device__ __forceinline__ float quotient(float x, const TileScale& t) {
  if constexpr (RULE == 0) {
    return div_by_scale(x * t.pre, t.d, t.y);
  } else {
    return x * t.y;
  }
}

// x / s for 8 values with one scale per lane.  Under the amax rule the
// pre-scaling multiply is skipped when no active lane of the wave has a tiny
// scale (a wave-uniform branch; there it is a multiply by 1).
template <int RULE>
__device__ __forceinline__ void quotient8(float (&v)[8], const TileScale& t) {
  if constexpr (RULE == 0) {
    if (__builtin_amdgcn_ballot_w64(t.pre != 1.0f) == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = div_by_scale(v[i], t.d, t.y);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = div_by_scale(v[i] * t.pre, t.d, t.y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * t.y;
  }
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
