// Shared device helpers of the gfx950 NVFP4 MoE library: the NVFP4 codecs in
// FP32 register arithmetic, wavefront reductions, and host-side argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4moe.h"

namespace nvfp4moe {

constexpr int kWave = 64;

// ------------------------------------------------------------------ codecs
// E4M3fn code of a finite v >= 0: nearest with ties to even, saturating at 448.
// Below 2^-6 the grid is the subnormal one (steps of 2^-9); v * 512 is exact and
// rint() rounds half to even, and the count 8 is code 0x08 (= 2^-6), so the
// subnormal and normal codes join up.  Above, the float32 significand is
// rounded to 3 bits (round half to even on the 20 dropped bits); a carry moves
// into the exponent field, which is the right next binade.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  return (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);   // biased exp: (e - 127) + 7
}

// E4M3fn code (non-negative, finite) -> float.
__device__ __forceinline__ float e4m3_decode_nonneg(uint32_t b) {
  uint32_t e = b >> 3, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Eight ratios -> eight E2M1 codes packed into one word (element j at bits
// 4j..4j+3) with v_cvt_scalef32_pk_fp4_f32, scale 1.0: nearest grid value of
// |r| in {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even grid index, saturating
// at 6, sign bit of r in bit 3.  (The quantiser's GPU tests compare its codes
// with the definition on every bf16 value up to 6 as an exact ratio, which
// covers each tie and its neighbours, and on random rows.)
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&r)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[0], r[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[2], r[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[4], r[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, r[6], r[7], 1.0f, 3);
  return w;
}

// ------------------------------------------------------------------ wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// double -> bf16 bits rounded once (nearest, ties to even), finite inputs.
// Rounds the float64 significand to 8 bits directly, then narrows exactly.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  double a = __builtin_fabs(d);
  if (a == 0.0) return (uint32_t)(__double_as_longlong(d) >> 48) & 0x8000u;
  int e;
  (void)__builtin_frexp(a, &e);            // a = m 2^e, m in [0.5, 1)
  if (e < -125) e = -125;                  // fixed step 2^-133 below 2^-126
  // a / 2^(e-8) and back: exact scalings by powers of two
  double r = __builtin_ldexp(__builtin_rint(__builtin_ldexp(a, 8 - e)), e - 8);
  float f = (float)r;                      // exact (<= 8 significant bits) or inf
  uint32_t bits = __float_as_uint(f) >> 16;
  return bits | (d < 0.0 ? 0x8000u : 0u);
}

// ------------------------------------------------------------------ float64 SwiGLU helpers
// 1/d for float64 d >= 1 (or +inf, or NaN): the hardware estimate refined by
// two Newton steps (the relative error squares at each step), within an ulp or
// so of the quotient; 1/inf = 0; NaN propagates.  It replaces a float64
// division where a result is rounded on to bf16: a few float64 ulps move the
// bf16 result only next to a bf16 rounding midpoint.
__device__ __forceinline__ double recip_f64(double d) {
  if (!(d < __builtin_inf())) return d != d ? d : 0.0;
  double y = __builtin_amdgcn_rcp(d);
  double e = __builtin_fma(-d, y, 1.0);
  y = __builtin_fma(y, e, y);
  e = __builtin_fma(-d, y, 1.0);
  return __builtin_fma(y, e, y);
}

// ------------------------------------------------------------------ host helpers
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

}  // namespace nvfp4moe
