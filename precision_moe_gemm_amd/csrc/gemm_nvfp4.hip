// Grouped NVFP4 (W4A4) expert GEMM for gfx950.
//
// The grouped GEMMs are where the miniTE pages locate the MoE cost of native
// FP4 (news.hamidun.com, "miniTE accélère le RL en NVFP4 sur B300",
// §Diagnostic, alignement et noyaux rapides); the operands live in contiguous
// expert-grouped buffers with device-side offsets (blog "miniTE NVFP4",
// §Two complementary interventions), so the kernel walks the experts' row
// ranges itself and the host never reads the routing.
//
// Exactness.  An element is e2m1(q) * e4m3(b) * s.  The product q*b has at
// most 6 significant bits and lies in [2^-10, 2688], so it is exact in FP16;
// the FP16 matrix cores multiply such pairs exactly and accumulate in FP32.
// The two FP32 row scales are applied once, in the epilogue.  (The gfx950
// block-scaled FP4 MFMA takes one power-of-two scale per 32 elements and
// cannot carry an E4M3 scale per 16 elements exactly.)
//
// Structure.  Workgroup tile 128x128 (rows of one expert x output columns),
// K-step 128, 4 wavefronts each owning 64x64 = 4x4 MFMA 16x16x32 tiles.
// Per K-step the FP4 codes (64 B per row) and E4M3 scales (8 B per row) of
// both operands are staged in LDS (double buffered, rows padded to 80 B so
// 16-byte reads from 16 rows hit distinct banks); each wavefront reads its
// 16-byte fragment (32 elements) per 16 rows and decodes it in registers with
// v_cvt_scalef32_pk_f16_fp4 and a packed FP16 multiply by the block scale.
// A lane of K-group g takes the 32 elements [32g, 32g+32) of the K-step and
// feeds 8 of them to each of 4 MFMAs; A and B use the same assignment, so the
// sum over K is complete (only its order differs, and that order does not
// depend on the number of rows).
// The grid is persistent: each workgroup walks tiles of a contiguous range
// owned by its XCD (workgroups go to the 8 XCDs round-robin), m-tile major,
// so the A rows and an expert's weights are reused from that XCD's L2.
#include "common.h"

namespace nvfp4moe {
namespace g4 {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kCodeBytes = BK / 2;           // 64 code bytes per row per K-step
constexpr int kStride = kCodeBytes + 16;     // padded LDS row
constexpr int kScaleBytes = BK / 16;         // 8 scale bytes per row per K-step

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct __align__(16) Stage {
  uint8_t a[BM * kStride];
  uint8_t w[BN * kStride];
  uint8_t as[BM * kScaleBytes];
  uint8_t ws[BN * kScaleBytes];
};

__device__ __forceinline__ half2v scale2(uint32_t b) {
  const _Float16 h = (_Float16)e4m3_decode_nonneg(b);   // exact: every E4M3 value is an FP16 value
  return half2v{h, h};
}

// 8 consecutive E2M1 codes (one 32-bit word, element 0 in the low nibble) -> 8 FP16 values q*b.
__device__ __forceinline__ half8 decode8(uint32_t w, half2v b2) {
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * b2;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * b2;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * b2;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * b2;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_bscales,
    const float* __restrict__ a_rscales, const int32_t* __restrict__ offsets, int E,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_bscales,
    const float* __restrict__ w_rscales, int N, int K, float* __restrict__ c) {
  __shared__ Stage st[2];
  __shared__ int tile_start[NVFP4MOE_MAX_EXPERTS + 1];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, g = lane >> 4;

  // m-tiles per expert -> exclusive prefix (device-side metadata only)
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
  // XCD-contiguous tile ranges when the grid is a multiple of 8 workgroups
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

  const int kb = K / 2, ks = K / 16, nk = K / BK;
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

    // global source of this thread's loads (rows clamped into the valid range)
    const uint8_t* ga[2];
    const uint8_t* gw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int chunk = tid + i * kThreads, row = chunk >> 2, part = chunk & 3;
      const int ar = min(m0 + row, m_end - 1);
      const int wr = min(n0 + row, N - 1);
      ga[i] = a_codes + (int64_t)ar * kb + part * 16;
      gw[i] = w_codes + ((int64_t)e * N + wr) * kb + part * 16;
    }
    const int ldsoff0 = (tid >> 2) * kStride + (tid & 3) * 16;
    const int ldsoff1 = ((tid + kThreads) >> 2) * kStride + (tid & 3) * 16;
    const uint8_t* gsc = tid < BM
        ? a_bscales + (int64_t)min(m0 + tid, m_end - 1) * ks
        : w_bscales + ((int64_t)e * N + min(n0 + tid - BM, N - 1)) * ks;

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    uint4 pa0, pa1, pw0, pw1;
    uint2 psc;
#define G4_GLOAD(kt)                                                              \
    pa0 = *reinterpret_cast<const uint4*>(ga[0] + (kt) * kCodeBytes);             \
    pa1 = *reinterpret_cast<const uint4*>(ga[1] + (kt) * kCodeBytes);             \
    pw0 = *reinterpret_cast<const uint4*>(gw[0] + (kt) * kCodeBytes);             \
    pw1 = *reinterpret_cast<const uint4*>(gw[1] + (kt) * kCodeBytes);             \
    psc = *reinterpret_cast<const uint2*>(gsc + (kt) * kScaleBytes);
#define G4_LSTORE(S)                                                              \
    *reinterpret_cast<uint4*>((S).a + ldsoff0) = pa0;                             \
    *reinterpret_cast<uint4*>((S).a + ldsoff1) = pa1;                             \
    *reinterpret_cast<uint4*>((S).w + ldsoff0) = pw0;                             \
    *reinterpret_cast<uint4*>((S).w + ldsoff1) = pw1;                             \
    *reinterpret_cast<uint2*>((tid < BM ? (S).as : (S).ws) + (tid & (BM - 1)) * kScaleBytes) = psc;

    G4_GLOAD(0)
    G4_LSTORE(st[0])
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const Stage& S = st[kt & 1];
      if (kt + 1 < nk) { G4_GLOAD(kt + 1) }
      uint32_t ra[4][4], rb[4][4];
      half2v sa[4][2], sb[4][2];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int arow = wm * 64 + f * 16 + l16;
        const int brow = wn * 64 + f * 16 + l16;
        const uint4 va = *reinterpret_cast<const uint4*>(S.a + arow * kStride + g * 16);
        const uint4 vb = *reinterpret_cast<const uint4*>(S.w + brow * kStride + g * 16);
        ra[f][0] = va.x; ra[f][1] = va.y; ra[f][2] = va.z; ra[f][3] = va.w;
        rb[f][0] = vb.x; rb[f][1] = vb.y; rb[f][2] = vb.z; rb[f][3] = vb.w;
        const uint32_t xa = *reinterpret_cast<const uint16_t*>(S.as + arow * kScaleBytes + 2 * g);
        const uint32_t xb = *reinterpret_cast<const uint16_t*>(S.ws + brow * kScaleBytes + 2 * g);
        sa[f][0] = scale2(xa & 0xFF); sa[f][1] = scale2(xa >> 8);
        sb[f][0] = scale2(xb & 0xFF); sb[f][1] = scale2(xb >> 8);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8 av[4], bv[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          av[f] = decode8(ra[f][s], sa[f][s >> 1]);
          bv[f] = decode8(rb[f][s], sb[f][s >> 1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) { G4_LSTORE(st[(kt + 1) & 1]) }
      __syncthreads();
    }
#undef G4_GLOAD
#undef G4_LSTORE

    // epilogue: C = (acc * s_A[row]) * s_W[col]; lane holds column l16 of each
    // 16x16 tile and rows 4g..4g+3.
    float swv[4];
    int ncol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ncol[j] = n0 + wn * 64 + j * 16 + l16;
      swv[j] = ncol[j] < N ? w_rscales[(int64_t)e * N + ncol[j]] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = m0 + wm * 64 + i * 16 + 4 * g + v;
        if (r < m_end) {
          const float sav = a_rscales[r];
          float* crow = c + (int64_t)r * N;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (ncol[j] < N) crow[ncol[j]] = (acc[i][j][v] * sav) * swv[j];
        }
      }
    }
  }
}

}  // namespace g4
}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" NVFP4MOE_API int nvfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_bscales,
                                               const float* a_rscales,
                                               const int32_t* expert_offsets, int32_t E,
                                               int64_t R_cap, const uint8_t* w_codes,
                                               const uint8_t* w_bscales, const float* w_rscales,
                                               int64_t N, int64_t K, float* c, void* stream) {
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS || R_cap < 0) return NVFP4_ERR_SHAPE;
  if (K <= 0 || K % g4::BK != 0 || K > 65536 || N < 16 || N % 16 != 0 || N > (1 << 24))
    return NVFP4_ERR_SHAPE;
  if (R_cap > INT32_MAX / 2 || (int64_t)E * N > INT32_MAX) return NVFP4_ERR_SHAPE;
  if (R_cap == 0) return NVFP4_OK;
  if (!a_codes || !a_bscales || !a_rscales || !expert_offsets || !w_codes || !w_bscales ||
      !w_rscales || !c)
    return NVFP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_bscales) || !aligned16(a_rscales) ||
      !aligned16(w_codes) || !aligned16(w_bscales) || !aligned16(w_rscales) || !aligned16(c))
    return NVFP4_ERR_ALIGN;
  const int64_t n_tiles = (N + g4::BN - 1) / g4::BN;
  const int64_t max_tiles = ((R_cap + g4::BM - 1) / g4::BM + E) * n_tiles;
  if (max_tiles > INT32_MAX) return NVFP4_ERR_SHAPE;
  // persistent grid: two workgroups per CU on a 256-CU device, a multiple of 8
  int64_t grid = max_tiles < 512 ? max_tiles : 512;
  if (grid >= 8) grid &= ~7ll;
  hipStream_t s = static_cast<hipStream_t>(stream);
  g4::grouped_gemm_kernel<<<(unsigned)grid, g4::kThreads, 0, s>>>(
      a_codes, a_bscales, a_rscales, expert_offsets, E, w_codes, w_bscales, w_rscales, (int)N,
      (int)K, c);
  return launch_status();
}
