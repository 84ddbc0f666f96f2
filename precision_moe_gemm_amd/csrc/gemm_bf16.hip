// BF16 grouped expert GEMM for the backward pass (input gradient), gfx950.
//
// The miniTE learner runs that are timed pair the NVFP4 forward with a BF16
// backward, and forward/backward precision are chosen independently (blog
// "miniTE NVFP4", yuxiaoba.github.io, §Respect the timing boundaries and §Two
// complementary interventions).  The input gradient of an expert GEMM
// C = A W_e^T is dA = dC W_e, a contraction over W's output dimension, so the
// weight is read in its stored [E][out][in] = [E][K][N] layout (NVFP4MOE_W_KN),
// i.e. with N contiguous.  NVFP4MOE_W_NK ([E][N][K]) is also accepted.
//
// Structure: 128x128 workgroup tile over one expert's rows, K-step 32 (one
// MFMA depth), 4 wavefronts of 64x64 (4x4 v_mfma_f32_16x16x32_bf16).  A and
// a [N][K] weight are staged as 64-byte rows (padded to 80 B) and read as
// 16-byte fragments.  A [K][N] weight is transposed while it is written to
// LDS: each thread loads rows k, k+1 of 8 columns and writes the 8 (k, k+1)
// pairs as 32-bit words into a [N][K] layout with 72-byte rows, which puts the
// 32 lanes of one write in 32 distinct banks; the fragment is then read as
// two 8-byte halves.  Tiles are scheduled like the NVFP4 GEMM: persistent
// workgroups, XCD-contiguous ranges, expert rows found from device offsets.
#include "common.h"

namespace nvfp4moe {
namespace gb {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int kThreads = 256;
constexpr int kRowBytes = BK * 2;            // 64
constexpr int kStride = kRowBytes + 16;      // 80: [rows][K] tiles
constexpr int kStrideT = kRowBytes + 8;      // 72: transposed weight tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <bool KN>
__global__ __launch_bounds__(kThreads, 2) void bf16_grouped_gemm_kernel(
    const uint16_t* __restrict__ a, const int32_t* __restrict__ offsets, int E,
    const uint16_t* __restrict__ w, int N, int K, float* __restrict__ c) {
  __shared__ __align__(16) uint8_t sa[2][BM * kStride];
  __shared__ __align__(16) uint8_t sw[2][BN * (KN ? kStrideT : kStride)];
  __shared__ int tile_start[NVFP4MOE_MAX_EXPERTS + 1];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, g = lane >> 4;

  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int v = e < E ? (offsets[e + 1] - offsets[e] + BM - 1) / BM : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      if (e < E) tile_start[e] = carry + incl - v;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) tile_start[E] = carry;
  }
  __syncthreads();

  const int n_tiles = (N + BN - 1) / BN;
  const int total = tile_start[E] * n_tiles;
  int begin, end, step;
  if ((gridDim.x & 7) == 0) {
    const int per = (total + 7) / 8;
    const int xcd = blockIdx.x & 7;
    begin = xcd * per + (int)(blockIdx.x >> 3);
    end = min(total, (xcd + 1) * per);
    step = gridDim.x >> 3;
  } else {
    begin = blockIdx.x;
    end = total;
    step = gridDim.x;
  }
  const int nk = K / BK;

  for (int L = begin; L < end; L += step) {
    const int tm = L / n_tiles, tn = L - tm * n_tiles;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_start[mid] <= tm) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int m_end = offsets[e + 1];
    const int m0 = offsets[e] + (tm - tile_start[e]) * BM;
    const int n0 = tn * BN;

    // A: chunks tid and tid+256 of the 128 x 64 B tile
    const uint16_t* ga0 = a + (int64_t)min(m0 + (tid >> 2), m_end - 1) * K + (tid & 3) * 8;
    const uint16_t* ga1 = a + (int64_t)min(m0 + 64 + (tid >> 2), m_end - 1) * K + (tid & 3) * 8;
    const int lo0 = (tid >> 2) * kStride + (tid & 3) * 16;
    const int lo1 = (64 + (tid >> 2)) * kStride + (tid & 3) * 16;
    // W
    const uint16_t* gw0;
    const uint16_t* gw1;
    int wl0 = 0, wl1 = 0;
    const int kp = tid & 15, ng = tid >> 4;               // KN: k pair, group of 8 columns
    if (KN) {
      const int col = min(n0 + ng * 8, N - 8);
      gw0 = w + (int64_t)e * K * N + (int64_t)(2 * kp) * N + col;
      gw1 = gw0 + N;
    } else {
      gw0 = w + ((int64_t)e * N + min(n0 + (tid >> 2), N - 1)) * K + (tid & 3) * 8;
      gw1 = w + ((int64_t)e * N + min(n0 + 64 + (tid >> 2), N - 1)) * K + (tid & 3) * 8;
      wl0 = lo0;
      wl1 = lo1;
    }

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    uint4 pa0, pa1, pw0, pw1;
#define GB_GLOAD(kt)                                                                   \
    pa0 = *reinterpret_cast<const uint4*>(ga0 + (kt) * BK);                            \
    pa1 = *reinterpret_cast<const uint4*>(ga1 + (kt) * BK);                            \
    if (KN) {                                                                          \
      pw0 = *reinterpret_cast<const uint4*>(gw0 + (int64_t)(kt) * BK * N);             \
      pw1 = *reinterpret_cast<const uint4*>(gw1 + (int64_t)(kt) * BK * N);             \
    } else {                                                                           \
      pw0 = *reinterpret_cast<const uint4*>(gw0 + (kt) * BK);                          \
      pw1 = *reinterpret_cast<const uint4*>(gw1 + (kt) * BK);                          \
    }
#define GB_LSTORE(buf)                                                                 \
    *reinterpret_cast<uint4*>(sa[buf] + lo0) = pa0;                                    \
    *reinterpret_cast<uint4*>(sa[buf] + lo1) = pa1;                                    \
    if (KN) {                                                                          \
      const uint32_t r0[4] = {pw0.x, pw0.y, pw0.z, pw0.w};                             \
      const uint32_t r1[4] = {pw1.x, pw1.y, pw1.z, pw1.w};                             \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                  \
        const uint32_t lo_pair = (r0[j] & 0xFFFFu) | (r1[j] << 16);                    \
        const uint32_t hi_pair = (r0[j] >> 16) | (r1[j] & 0xFFFF0000u);                \
        *reinterpret_cast<uint32_t*>(sw[buf] + (ng * 8 + 2 * j) * kStrideT + kp * 4) = lo_pair;     \
        *reinterpret_cast<uint32_t*>(sw[buf] + (ng * 8 + 2 * j + 1) * kStrideT + kp * 4) = hi_pair; \
      }                                                                                \
    } else {                                                                           \
      *reinterpret_cast<uint4*>(sw[buf] + wl0) = pw0;                                  \
      *reinterpret_cast<uint4*>(sw[buf] + wl1) = pw1;                                  \
    }

    GB_GLOAD(0)
    GB_LSTORE(0)
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) { GB_GLOAD(kt + 1) }
      bf16x8 av[4], bv[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int arow = wm * 64 + f * 16 + l16;
        const int brow = wn * 64 + f * 16 + l16;
        av[f] = *reinterpret_cast<const bf16x8*>(sa[cur] + arow * kStride + g * 16);
        if (KN) {
          const uint2 h0 = *reinterpret_cast<const uint2*>(sw[cur] + brow * kStrideT + g * 16);
          const uint2 h1 = *reinterpret_cast<const uint2*>(sw[cur] + brow * kStrideT + g * 16 + 8);
          const uint4 v = make_uint4(h0.x, h0.y, h1.x, h1.y);
          bv[f] = *reinterpret_cast<const bf16x8*>(&v);
        } else {
          bv[f] = *reinterpret_cast<const bf16x8*>(sw[cur] + brow * kStride + g * 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
      if (kt + 1 < nk) { GB_LSTORE(cur ^ 1) }
      __syncthreads();
    }
#undef GB_GLOAD
#undef GB_LSTORE

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = m0 + wm * 64 + i * 16 + 4 * g + v;
        if (r < m_end) {
          float* crow = c + (int64_t)r * N;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + l16;
            if (n < N) crow[n] = acc[i][j][v];
          }
        }
      }
    }
  }
}

}  // namespace gb
}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" NVFP4MOE_API int bf16_grouped_gemm(const uint16_t* a, const int32_t* expert_offsets,
                                              int32_t E, int64_t R_cap, const uint16_t* w,
                                              int32_t w_layout, int64_t N, int64_t K, float* c,
                                              void* stream) {
  if (w_layout != NVFP4MOE_W_KN && w_layout != NVFP4MOE_W_NK) return NVFP4_ERR_ARG;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS || R_cap < 0) return NVFP4_ERR_SHAPE;
  if (K <= 0 || K % gb::BK != 0 || N < 16 || N % 16 != 0) return NVFP4_ERR_SHAPE;
  if (R_cap * K > INT32_MAX * 8ll || (int64_t)E * N * K > (1ll << 40) || N > (1 << 24) ||
      K > (1 << 24) || R_cap > INT32_MAX / 2)
    return NVFP4_ERR_SHAPE;
  if (R_cap == 0) return NVFP4_OK;
  if (!a || !expert_offsets || !w || !c) return NVFP4_ERR_NULL;
  if (!aligned16(a) || !aligned16(w) || !aligned16(c)) return NVFP4_ERR_ALIGN;
  const int64_t n_tiles = (N + gb::BN - 1) / gb::BN;
  const int64_t max_tiles = ((R_cap + gb::BM - 1) / gb::BM + E) * n_tiles;
  if (max_tiles > INT32_MAX) return NVFP4_ERR_SHAPE;
  int64_t grid = max_tiles < 512 ? max_tiles : 512;
  if (grid >= 8) grid &= ~7ll;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_layout == NVFP4MOE_W_KN)
    gb::bf16_grouped_gemm_kernel<true><<<(unsigned)grid, gb::kThreads, 0, s>>>(
        a, expert_offsets, E, w, (int)N, (int)K, c);
  else
    gb::bf16_grouped_gemm_kernel<false><<<(unsigned)grid, gb::kThreads, 0, s>>>(
        a, expert_offsets, E, w, (int)N, (int)K, c);
  return launch_status();
}
