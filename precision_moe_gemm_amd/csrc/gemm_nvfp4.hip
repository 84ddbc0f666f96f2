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
// Structure.  Workgroup tile 128 x 512 (rows of one expert x output columns),
// K-step 128, 8 wavefronts (two per SIMD, so one wavefront's decode and LDS
// traffic hide under the other's MFMAs), each owning 128 x 64 outputs as 8 x 4
// MFMA 16x16x32 tiles (accumulators in AGPRs).  The MFMA computes C^T tiles
// (weights as its first operand), which leaves 4 consecutive output columns in
// each lane for 16-byte stores.
//   * FP4 codes (64 B per row per K-step) and E4M3 scales (8 B per row) of both
//     operands go from global memory straight into LDS (global_load_lds,
//     two stages, no staging registers); code rows are stored as four 16-byte
//     chunks XOR-swizzled by row, so 16-byte reads of 8 consecutive rows fall
//     in distinct banks.
//   * The activation tile is shared by all 8 wavefronts, so it is decoded once
//     per K-step, cooperatively, into an FP16 tile in LDS (256 B rows, 16-byte
//     chunks XOR-swizzled by row); each wavefront decodes only its own weight
//     fragments, in registers, interleaved with its MFMAs.
//   * Decoding is v_cvt_scalef32_pk_f16_fp4 plus one packed FP16 multiply by
//     the block scale per element pair.
// A lane of K-group g takes the 32 elements [32g, 32g+32) of the K-step and
// feeds 8 of them to each of 4 MFMA K-slices; both operands use the same
// assignment, so the sum over K is complete and its order does not depend on
// the number of rows.
// The grid is persistent: each workgroup walks tiles of a contiguous range
// owned by its XCD (workgroups go to the 8 XCDs round-robin), m-tile major,
// so the A rows and an expert's weights are reused from that XCD's L2.
#include "common.h"

namespace nvfp4moe {
namespace g4 {

constexpr int BM = 128, BN = 512, BK = 128;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowB = BK / 2;                // 64 code bytes per row per K-step
constexpr int kScB = BK / 16;                // 8 scale bytes per row per K-step
constexpr int WN = BN / kWaves;              // 64 columns per wavefront
constexpr int FA = BM / 16, FB = WN / 16;    // 8 x 4 MFMA tiles per wavefront
constexpr int kA16Row = BK * 2;              // 256 B per row of the decoded activation tile

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

struct __align__(16) Stage {
  uint8_t a[BM * kRowB];       // 8 KiB FP4 activation codes
  uint8_t w[BN * kRowB];       // 32 KiB FP4 weight codes
  uint8_t as[BM * kScB];       // 1 KiB
  uint8_t ws[BN * kScB];       // 4 KiB
};

struct __align__(16) Smem {
  Stage st[2];
  uint8_t a16[2][BM * kA16Row];   // 2 x 32 KiB decoded activations (FP16)
  int tile_start[NVFP4MOE_MAX_EXPERTS + 1];
};

// physical 16-byte chunk of logical chunk c in row r of an FP4 code tile
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }
// byte offset of 16-byte chunk c (0..15) of row r in the FP16 activation tile
__device__ __forceinline__ int a16_off(int r, int c) { return r * kA16Row + ((c ^ (r & 7)) << 4); }

// E4M3 byte b (non-negative) -> two FP16 copies of b * 2^-8.  The 7 value bits
// of E4M3 shifted up by 7 land exactly on FP16's exponent/mantissa fields with
// the exponent bias off by 8 (15 - 7), for normal and subnormal codes alike.
__device__ __forceinline__ uint32_t scale_pair(uint32_t b) { return b * 0x00800080u; }

// 8 consecutive E2M1 codes (one word, element 0 in the low nibble) -> 8 FP16
// values q*b.  The convert's scale operand only contributes its exponent, so it
// carries the 2^8 and the packed multiply carries b * 2^-8: the product is
// exact (at most 6 significant bits, within FP16's normal range).
__device__ __forceinline__ half8 decode8(uint32_t w, uint32_t sp) {
  const half2v s2 = __builtin_bit_cast(half2v, sp);
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s2;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s2;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s2;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s2;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t word(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_bscales,
    const float* __restrict__ a_rscales, const int32_t* __restrict__ offsets, int E,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_bscales,
    const float* __restrict__ w_rscales, int N, int K, float* __restrict__ c) {
  __shared__ Smem sm;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
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
      if (e < E) sm.tile_start[e] = carry + incl - v;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) sm.tile_start[E] = carry;
  }
  __syncthreads();

  const int n_tiles = (N + BN - 1) / BN;
  const int total = sm.tile_start[E] * n_tiles;
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
  // cooperative activation decode: lane -> row 16*wave + lane/4, K quarter lane%4
  const int drow = 16 * wave + (lane >> 2), dq = lane & 3;

  for (int L = begin; L < end; L += step) {
    const int tm = L / n_tiles, tn = L - tm * n_tiles;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm.tile_start[mid] <= tm) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int m_end = offsets[e + 1];
    const int m0 = offsets[e] + (tm - sm.tile_start[e]) * BM;
    const int n0 = tn * BN;

    // Sources of this lane's direct-to-LDS loads, as 32-bit byte offsets from
    // the operand bases (the host keeps every operand under 4 GiB).  A
    // wavefront instruction fills 1 KiB of LDS (16 rows of codes; lane l ->
    // row l/4, physical chunk l%4), so the lane loads the logical chunk that
    // belongs in that slot.  Wavefront w loads code rows [16w, 16w+16) of A
    // and rows 128j + [16w, 16w+16) of W; scale dwords go one per lane.
    uint32_t off_a, off_w[4], off_s[3];
    {
      const int row = 16 * wave + (lane >> 2);
      const int chunk = (lane & 3) ^ swz(row);
      off_a = (uint32_t)min(m0 + row, m_end - 1) * (uint32_t)kb + chunk * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        off_w[j] = ((uint32_t)e * N + min(n0 + 128 * j + row, N - 1)) * (uint32_t)kb + chunk * 16;
      // scale dwords: 1280 in all (A: 256, W: 1024); dword d -> row d/2, half d%2
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int d = 512 * j + tid;
        if (d < 256)
          off_s[j] = (uint32_t)min(m0 + (d >> 1), m_end - 1) * (uint32_t)ks + (d & 1) * 4;
        else
          off_s[j] = ((uint32_t)e * N + min(n0 + ((d - 256) >> 1), N - 1)) * (uint32_t)ks + (d & 1) * 4;
      }
    }

#define G4_ISSUE_LOADS(kt, S)                                                                      \
    {                                                                                              \
      __builtin_amdgcn_global_load_lds((glb_void*)(a_codes + (kt) * kRowB + off_a),                \
                                       (lds_void*)((S).a + wave * 1024), 16, 0, 0);                \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                \
        __builtin_amdgcn_global_load_lds((glb_void*)(w_codes + (kt) * kRowB + off_w[j]),           \
                                         (lds_void*)((S).w + (8 * j + wave) * 1024), 16, 0, 0);    \
      /* scale dwords 0..255 -> as, 256..1279 -> ws (as and ws are adjacent) */                   \
      _Pragma("unroll") for (int j = 0; j < 3; ++j) {                                              \
        const int d0 = 512 * j + 64 * wave;                                                        \
        if (d0 < 1280) {                                                                           \
          const uint8_t* base = d0 < 256 ? a_bscales : w_bscales;                                  \
          __builtin_amdgcn_global_load_lds((glb_void*)(base + (kt) * kScB + off_s[j]),             \
                                           (lds_void*)((S).as + d0 * 4), 4, 0, 0);                 \
        }                                                                                          \
      }                                                                                            \
    }

    // decode this lane's share of the activation tile of a stage into an FP16 tile:
    // row drow, elements [32 dq, 32 dq + 32) = logical FP4 chunk dq, block scales 2dq, 2dq+1
#define G4_DECODE_A(S, A16)                                                                        \
    {                                                                                              \
      const uint4 v = *reinterpret_cast<const uint4*>((S).a + drow * kRowB + ((dq ^ swz(drow)) << 4)); \
      const uint32_t x = *reinterpret_cast<const uint16_t*>((S).as + drow * kScB + 2 * dq);        \
      const uint32_t s0 = scale_pair(x & 0xFF), s1 = scale_pair(x >> 8);                           \
      const half8 h0 = decode8(v.x, s0), h1 = decode8(v.y, s0);                                    \
      const half8 h2 = decode8(v.z, s1), h3 = decode8(v.w, s1);                                    \
      *reinterpret_cast<half8*>((A16) + a16_off(drow, 4 * dq + 0)) = h0;                           \
      *reinterpret_cast<half8*>((A16) + a16_off(drow, 4 * dq + 1)) = h1;                           \
      *reinterpret_cast<half8*>((A16) + a16_off(drow, 4 * dq + 2)) = h2;                           \
      *reinterpret_cast<half8*>((A16) + a16_off(drow, 4 * dq + 3)) = h3;                           \
    }

    floatx4 acc[FA][FB];
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
      for (int j = 0; j < FB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // prologue: K-step 0 loaded and decoded, K-step 1 in flight
    G4_ISSUE_LOADS(0, sm.st[0])
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    G4_DECODE_A(sm.st[0], sm.a16[0])
    if (nk > 1) G4_ISSUE_LOADS(1, sm.st[1])
    __syncthreads();

    // raw weight fragments of the K-step (4 slices in a 16-byte read) and scales
    uint4 rb[FB];
    uint32_t xb[FB];
#define G4_READ_B(S)                                                                               \
    _Pragma("unroll") for (int f = 0; f < FB; ++f) {                                               \
      const int row = wave * WN + f * 16 + l16;                                                    \
      rb[f] = *reinterpret_cast<const uint4*>((S).w + row * kRowB + ((g ^ swz(row)) << 4));        \
      xb[f] = *reinterpret_cast<const uint16_t*>((S).ws + row * kScB + 2 * g);                     \
    }
    G4_READ_B(sm.st[0])

    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* A16 = sm.a16[kt & 1];
      // MFMA D = W_frag x A_frag^T: C^T tiles.  Activation fragments come
      // decoded from LDS (16-byte reads); the weight fragments of slice s+1
      // are decoded in registers while slice s runs on the matrix cores.
      half8 bv[FB], bn[FB];
#pragma unroll
      for (int j = 0; j < FB; ++j) bv[j] = decode8(rb[j].x, scale_pair(xb[j] & 0xFF));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < FA; ++i) {
          const half8 av = *reinterpret_cast<const half8*>(A16 + a16_off(i * 16 + l16, 4 * g + s));
          if (s + 1 < 4 && i < FB)
            bn[i] = decode8(word(rb[i], s + 1), scale_pair(s + 1 < 2 ? (xb[i] & 0xFF) : (xb[i] >> 8)));
#pragma unroll
          for (int j = 0; j < FB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv[j], av, acc[i][j], 0, 0, 0);
        }
        if (s + 1 < 4) {
#pragma unroll
          for (int j = 0; j < FB; ++j) bv[j] = bn[j];
        }
      }
      if (kt + 1 < nk) {
        const Stage& S1 = sm.st[(kt + 1) & 1];
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this lane's loads of K-step kt+1 landed
        __syncthreads();                      // everyone's; all reads of a16[kt&1] and stage kt&1 done
        G4_READ_B(S1)
        G4_DECODE_A(S1, sm.a16[(kt + 1) & 1])
        if (kt + 2 < nk) G4_ISSUE_LOADS(kt + 2, sm.st[kt & 1])
        __syncthreads();                      // decoded activations visible
      }
    }
#undef G4_ISSUE_LOADS
#undef G4_DECODE_A
#undef G4_READ_B

    // epilogue: C = (acc * s_A[row]) * s_W[col].  Tile (i, j) of the lane holds
    // row 16i + l16 and columns 16j + 4g .. 16j + 4g + 3: one 16-byte store.
    float4 swv[FB];
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      const int n = n0 + wave * WN + j * 16 + 4 * g;
      swv[j] = n < N ? *reinterpret_cast<const float4*>(w_rscales + (int64_t)e * N + n)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < FA; ++i) {
      const int r = m0 + i * 16 + l16;
      if (r < m_end) {
        const float sav = a_rscales[r];
        float* crow = c + (int64_t)r * N + n0 + wave * WN + 4 * g;
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          if (n0 + wave * WN + j * 16 + 4 * g < N) {
            float4 o;
            o.x = (acc[i][j][0] * sav) * swv[j].x;
            o.y = (acc[i][j][1] * sav) * swv[j].y;
            o.z = (acc[i][j][2] * sav) * swv[j].z;
            o.w = (acc[i][j][3] * sav) * swv[j].w;
            *reinterpret_cast<float4*>(crow + j * 16) = o;
          }
        }
      }
    }
    __syncthreads();   // the next tile's prologue overwrites stage 0 and a16[0]
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
  // the kernel addresses each operand with 32-bit byte offsets
  if (R_cap * (K / 2) > (int64_t)UINT32_MAX || (int64_t)E * N * (K / 2) > (int64_t)UINT32_MAX)
    return NVFP4_ERR_SHAPE;
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
  // persistent grid: one workgroup (8 wavefronts) per CU on a 256-CU device, a multiple of 8
  int64_t grid = max_tiles < 256 ? max_tiles : 256;
  if (grid >= 8) grid &= ~7ll;
  hipStream_t s = static_cast<hipStream_t>(stream);
  g4::grouped_gemm_kernel<<<(unsigned)grid, g4::kThreads, 0, s>>>(
      a_codes, a_bscales, a_rscales, expert_offsets, E, w_codes, w_bscales, w_rscales, (int)N,
      (int)K, c);
  return launch_status();
}
