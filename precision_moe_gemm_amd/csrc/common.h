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

// double -> bf16 bits rounded once (nearest, ties to even), non-NaN inputs.
// With e the binade of |d| clamped to [-126, 978], |d| + C for C = 2^(e+45)
// lies in C's binade, whose ulp 2^(e-7) is the bf16 step at |d| (below 2^-126
// the fixed subnormal step 2^-133), so (|d| + C) - C is |d| rounded once to
// 8 significant bits; it narrows to float exactly, or to inf past the bf16
// range.  The sign is d's, zeros included.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  const uint32_t hi = (uint32_t)((uint64_t)__double_as_longlong(d) >> 32);
  const uint32_t be = min(max((hi >> 20) & 0x7FFu, 897u), 2001u);   // biased exponent, clamped
  const double C = __longlong_as_double((long long)((uint64_t)((be + 45u) << 20) << 32));
  const double r = (__builtin_fabs(d) + C) - C;
  return (__float_as_uint((float)r) | (hi & 0x80000000u)) >> 16;
}

// ------------------------------------------------------------------ float64 SwiGLU helpers
// 2^(j/64) for j = 0..63, each the nearest double.
static __constant__ double kExp2Frac64[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

// Copies kExp2Frac64 into a workgroup's LDS table (blocks of at least 64
// threads).  Per-lane indexed reads of it then have a short latency and their
// own wait counter, where global reads would queue behind the row's loads.
// Holds a barrier: call it before any early return.
__device__ __forceinline__ void stage_exp2_table(double* tab) {
  if (threadIdx.x < 64) tab[threadIdx.x] = kExp2Frac64[threadIdx.x];
  __syncthreads();
}

// 1 / (1 + exp(-g)) in float64 for a float g, without a division and with a
// short exp (the SwiGLU kernels are bound by the issue of their float64 work);
// tab is the LDS copy of kExp2Frac64:
//  * x = -g is clamped to [-746, 710]: exp(x) stays 0 below (it is below half
//    the least subnormal there) and overflows to +inf above, as unclamped;
//  * x = k ln2/64 + r with k the nearest integer to 64 x / ln2, found by one
//    fma with 1.5 * 2^52 (whose low word is then k), and ln2/64 split in a
//    32-bit head (k * head is exact) and a tail, so |r| <= ln2/128;
//  * exp(r) by its Taylor polynomial of degree 5 (truncation below 2^-54
//    relative), times 2^((k & 63)/64) from the table, scaled by 2^(k >> 6);
//  * 1/d by the hardware estimate and two Newton steps (the error squares at
//    each step) taken on min(d, DBL_MAX), so that d = +inf gives exactly 0.
// The result is within 2^-50 relative of the exact sigmoid of g (a few
// float64 ulps); NaN propagates.
__device__ __forceinline__ double sigmoid_f64(float g, const double* tab) {
  const double x = (double)__builtin_amdgcn_fmed3f(-g, -746.0f, 710.0f);
  const double t = __builtin_fma(x, 0x1.71547652b82fep+6, 0x1.8p52);
  const int k = (int)(uint32_t)__double_as_longlong(t);
  const double kd = t - 0x1.8p52;
  double r = __builtin_fma(-kd, 0x1.62e42fee00000p-7, x);
  r = __builtin_fma(-kd, 0x1.a39ef35793c76p-39, r);
  double p = __builtin_fma(r, 0x1.1111111111111p-7, 0x1.5555555555555p-5);
  p = __builtin_fma(p, r, 0x1.5555555555555p-3);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  const double d = 1.0 + __builtin_ldexp(p * tab[k & 63], k >> 6);
  const double y0 = __builtin_amdgcn_rcp(d);
  const double dc = __builtin_fmin(d, 0x1.fffffffffffffp+1023);
  double y = __builtin_fma(y0, __builtin_fma(-dc, y0, 1.0), y0);
  return __builtin_fma(y, __builtin_fma(-dc, y, 1.0), y);
}

// ------------------------------------------------------------------ host helpers
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

}  // namespace nvfp4moe
