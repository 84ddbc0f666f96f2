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
// Structure.  One 512-thread workgroup per CU (about 157 KiB of LDS), two
// wavefronts per SIMD.  Workgroup tile 128 x 512 (rows of one expert x output
// columns), K-step 64; wavefront w owns the columns [64w, 64w+64) for all 128
// rows as 4 x 2 MFMA 32x32x16 tiles.  The MFMA computes C^T tiles (weights as
// its first operand), which leaves 4 consecutive output columns in each lane
// for 16-byte stores.
//   * FP4 codes (32 B per row per K-step) and E4M3 scales (4 B per row) of
//     both operands go from global memory straight into LDS
//     (global_load_lds) in a 3-stage ring: the loads of K-step g+3 are issued
//     when K-step g starts, two full K-steps before they are read.  With
//     K-tiled weights every wavefront issues the same three loads per K-step
//     from per-tile offsets (the weight block scales of a K-step are then
//     contiguous, 16 bytes = 4 rows per lane), so the issue has no branches
//     beyond one on the load width.
//   * The activation tile is shared by the 8 wavefronts, so it is decoded once
//     per K-step, cooperatively, into an FP16 tile in LDS (128 B rows, 16-byte
//     chunks XOR-swizzled by row pair); each wavefront decodes only its own weight
//     fragments, in registers.  Both decodes of K-step g+1 are interleaved with
//     the MFMAs of K-step g, so one barrier per K-step suffices.
//   * Decoding is v_cvt_scalef32_pk_f16_fp4 plus one packed FP16 multiply by
//     the block scale per element pair.
//   * A tile's epilogue runs after the first barrier of the next tile: its
//     output stores are issued after the loads that this K-step's wait needed,
//     so the first wait that covers them is the next K-step's, and they have a
//     whole K-step to drain.
// Lane half h (lanes 32h..32h+31) of every MFMA takes the elements
// [32h, 32h+32) of the K-step, i.e. block scales 2h and 2h+1, and feeds 8 of
// them to each of the 4 MFMA K-slices.  Both operands use the same
// assignment, so the sum over K is complete and its order does not depend on
// the number of rows (or on the tile the row lands in).
// Rows past an expert's end are never computed on: a tile with fewer than 128
// rows skips its empty 32-row fragments, and the epilogue's buffer stores are
// range-checked by the hardware against the tile's valid rows.
// The grid is persistent: each workgroup walks tiles of a contiguous range
// owned by its XCD (workgroups go to the 8 XCDs round-robin), m-tile major,
// so the A rows and an expert's weights are reused from that XCD's L2.
// Dense (one-group) launches split a last round that would keep at most a
// quarter of a range's workgroups busy into 128 x 128 quarter tiles, one per
// workgroup: wavefront w takes rows 64 (w / 4) .. + 63 and column group w % 4
// with the same MFMAs (so the same bits) as in a whole tile, and a quarter
// costs about three quarters of a whole tile (its loads, barriers and
// activation decode do not shrink).
#include "common.h"

#include <type_traits>

namespace nvfp4moe {
namespace g5 {

constexpr int BM = 128, BN = 512, BK = 64;
constexpr int kStages = 3;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowB = BK / 2;                // 32 code bytes per row per K-step
constexpr int kScB = BK / 16;                // 4 scale bytes per row per K-step
constexpr int WN = BN / kWaves;              // 64 columns per wavefront
constexpr int FA = BM / 32, FB = WN / 32;    // 4 x 2 MFMA 32x32 tiles per wavefront
// Load instructions per K-step (one wavefront instruction fills 1 KiB of LDS):
// codes of 32 rows each (activation rows first, then weight rows), and block
// scales (or, once per tile, row scales) of 64 rows each.
constexpr int kCI = (BM + BN) * kRowB / 1024;     // 20 code instructions
constexpr int kSI = (BM + BN) / 64;               // 10 scale instructions
constexpr int kCIW = (kCI + kWaves - 1) / kWaves; // per wavefront, at most
constexpr int kSIW = (kSI + kWaves - 1) / kWaves;
constexpr int kA16Row = BK * 2;              // 128 B per row of the decoded activation tile
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset that the range check drops
constexpr int kNonTemporal = 2;                 // buffer store cache policy: nt

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct __align__(16) Stage {
  uint8_t a[BM * kRowB];       // 4 KiB FP4 activation codes, row-major
  uint8_t w[BN * kRowB];       // 16 KiB FP4 weight codes (directly after a): per 32 rows, the
                               // first 16 bytes of each row, then the last 16 (16 B per row)
  uint8_t as[BM * kScB];       // 512 B
  uint8_t ws[BN * kScB];       // 2 KiB (directly after as)
};

constexpr int kMtCap = 8192;   // m-tiles whose expert the prologue tabulates in LDS

struct __align__(16) Smem {
  Stage st[kStages];
  uint8_t a16[2][BM * kA16Row];   // 2 x 16 KiB decoded activations (FP16)
  uint8_t stg[kWaves][4096];      // per-wavefront staging of one 32 x 32 FP32 output tile
  float rs[2][BM + BN];            // row scales of a tile's rows, then of its weight rows (epilogue)
  float rw[2][BM];                 // router weights of a tile's rows (SwiGLU epilogue)
  int tile_start[NVFP4MOE_MAX_EXPERTS + 1];   // m-tiles before expert e
  int16_t mt_expert[kMtCap];                  // expert of m-tile tm (when they fit)
};

// byte offset of 16-byte chunk c (0..7) of row r in the FP16 activation tile.
// An LDS pass serves 16 lanes of a 16-byte read; the fragment reads put rows
// r..r+15 (r a multiple of 16) in one pass.  The 64 four-byte banks span 256
// bytes, two 128-byte rows: even rows sit on one half of the banks, odd rows
// on the other, so the chunk index is XORed with (r / 2) mod 8 and the 16 rows
// fall on 16 distinct 16-byte bank groups (as do the decoder's writes: 4 rows
// x 4 chunks per pass).
__device__ __forceinline__ int a16_off(int r, int c) { return r * kA16Row + ((c ^ ((r >> 1) & 7)) << 4); }

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

// Workgroup barrier that orders LDS only: global memory (in particular the
// direct-to-LDS loads still in flight) is left alone, so the barrier does not
// wait for them; their completion is waited for explicitly with vmcnt.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Direct-to-LDS loads (global_load_lds): each lane's 16 (or 4) bytes at
// base + voff land at lds + 16 * lane (4 * lane).  Issued through inline
// assembly so that the compiler, which cannot tell which LDS bytes such a load
// writes, does not make every later LDS read wait for all of them; the kernel
// waits for them itself (vmcnt) before the barrier that publishes a stage.
// The compiler does not count these loads, so its own vmcnt waits for other
// loads only become stricter.  M0 is written here and nowhere else in the
// kernel (no other M0-using instruction is generated).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const uint8_t* base, uint32_t voff, const uint8_t* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const uint8_t* base, uint32_t voff, const uint8_t* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
// the same with the LDS destination given as a wave-uniform LDS byte address
__device__ __forceinline__ void lds_dma16_at(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_at(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds), "v"(voff), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt with expcnt and lgkmcnt at their maxima: vmcnt(n), n in {0, 3, 4, 5}
  if (n == 5) __builtin_amdgcn_s_waitcnt(0x0F75);
  else if (n == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
  else if (n == 3) __builtin_amdgcn_s_waitcnt(0x0F73);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// One tile: rows [m0, m0 + rows) of expert e (rows <= BM), columns [n0, n0 + BN),
// or, for a quarter tile (q = 0..3), columns [n0, n0 + BN / 4) with n0 the
// whole tile's first column + q BN / 4.
struct Tile {
  int e, m0, rows, n0;
  int kb0, nk;   // first K-step of the tile's contraction and its K-steps
  int q;         // -1: a whole tile; 0..3: a column quarter
};
constexpr int kQW = BN / 4;              // columns of a quarter tile
constexpr int kNoTile = 0x7fffffff;      // end of a workgroup's tile sequence

// the expert of m-tile tm: the last e with tile_start[e] <= tm
__device__ __forceinline__ int expert_of(int tm, const int* tile_start, int E) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= tm) lo = mid; else hi = mid;
  }
  return lo;
}

// mt_expert: the prologue's table of expert_of, or null when it did not fit
// Row groups: rows [offsets[e], offsets[e+1]) of group e, each offset clamped
// into [0, Rc] (the rows the buffers hold), so that malformed offsets give
// wrong rows but no access outside the buffers; with KG (K-grouped, the weight
// gradient) every group has Mg rows (offsets unused) and contracts over its own
// K-steps [kofs[e], kofs[e+1]), clamped into the nk K-steps of the operands.
template <bool KG>
__device__ __forceinline__ int group_off(const int32_t* __restrict__ offsets, int Mg, int e) {
  if constexpr (KG) return e * Mg;
  else return min(max(offsets[e], 0), Mg);
}

// Tile L < total is whole tile L; with QT, L >= total is quarter
// (L - total) % 4 of whole tile (L - total) / 4.
template <bool KG, bool QT>
__device__ __forceinline__ Tile tile_at(int L, int total, int n_tiles, const int* tile_start,
                                        const int16_t* mt_expert, int E,
                                        const int32_t* __restrict__ offsets, int Mg,
                                        const int32_t* __restrict__ kofs, int nk) {
  int q = -1;
  if constexpr (QT) {
    if (L >= total) {
      q = (L - total) & 3;
      L = (L - total) >> 2;
    }
  }
  const int tm = L / n_tiles, tn = L - tm * n_tiles;
  const int lo = mt_expert ? (int)mt_expert[tm] : expert_of(tm, tile_start, E);
  // the values are the same in every lane: keep them in scalar registers
  Tile t;
  t.e = __builtin_amdgcn_readfirstlane(lo);
  t.m0 = __builtin_amdgcn_readfirstlane(group_off<KG>(offsets, Mg, t.e) + (tm - tile_start[t.e]) * BM);
  t.rows = __builtin_amdgcn_readfirstlane(min(BM, group_off<KG>(offsets, Mg, t.e + 1) - t.m0));
  t.n0 = tn * BN + (q >= 0 ? q * kQW : 0);
  t.q = q;
  if constexpr (KG) {
    t.kb0 = __builtin_amdgcn_readfirstlane(min(max(kofs[t.e], 0), nk - 1));
    t.nk = __builtin_amdgcn_readfirstlane(min(max(kofs[t.e + 1] - t.kb0, 1), nk - t.kb0));
  } else {
    t.kb0 = 0;
    t.nk = nk;
  }
  return t;
}

// Weighted SwiGLU of one gate/up pair in FP32: h = (silu(g) * u) * w, with
// silu(g) = g / (1 + exp(-g)) formed as g * rcp(1 + exp2(-g log2(e))) from the
// hardware exp2 and reciprocal (about 1 ulp each).  Within a few FP32 ulps of
// the float64 value wherever |h| is not negligible next to the row's largest
// |h| (for g far below zero exp(-g) carries a relative error of about
// |g| 2^-24, while silu(g) is tiny); 1 + exp(-g) = inf gives silu = -0.
__device__ __forceinline__ float swiglu_f32(float g, float u, float w) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return ((g * __builtin_amdgcn_rcpf(1.0f + e)) * u) * w;
}

// KT: K-tiled weights; OB: BF16 output (each FP32 result rounded to nearest
// even); SW: the weighted SwiGLU epilogue of the gate_up GEMM (K-tiled weights
// [E][K/64][2I][32], gate rows [0, I), up rows [I, 2I); output h [R][I] FP32;
// optionally gu [R][2I] FP32, the values the plain GEMM would write).  For SW
// a tile covers h columns [256 tn, 256 tn + 256): wavefront w's column
// fragment 0 holds gate rows 256 tn + 32 w + (0..31) and fragment 1 the up rows
// I + 256 tn + 32 w + (0..31), so a lane holds g and u of the same (row,
// column) in acc[i][0] and acc[i][1].
// Mg: the row capacity R_cap of A and C (offsets are clamped into it), or with
// KG the rows of every group.
// KG: K-grouped (the weight gradient): group e is the Mg activation rows
// (row-major [Mg][K/2], K = the padded total of all groups' K-steps) times the
// K-tiled weights [K/64][N][32], both over the group's K-steps
// [kofs[e], kofs[e+1]); its output rows are e Mg .. e Mg + Mg - 1; row scales
// a_rscales [E][Mg], w_rscales [E][N].
template <bool KT, bool OB, bool SW, bool KG, bool QT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_bscales,
    const float* __restrict__ a_rscales, const int32_t* __restrict__ offsets, int E,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_bscales,
    const float* __restrict__ w_rscales, int N, int K, void* __restrict__ c,
    const float* __restrict__ w_rows, float* __restrict__ gu_out, int I,
    const int32_t* __restrict__ kofs, int Mg) {
  static_assert(!SW || (KT && !OB), "the SwiGLU epilogue reads K-tiled weights and writes FP32");
  static_assert(!KG || (KT && !SW), "K-grouped tiles read K-tiled weights");
  constexpr bool kQuarters = QT && !SW && !OB && !KG;   // quarter tiles (plain FP32 output only)
  __shared__ Smem sm;
  constexpr bool w_tiled = KT;

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;

  // m-tiles per expert -> exclusive prefix (device-side metadata only)
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int v = e < E ? max(0, group_off<KG>(offsets, Mg, e + 1) - group_off<KG>(offsets, Mg, e) + BM - 1) / BM
                          : 0;
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

  const int n_tiles = SW ? I / (BN / 2) : (N + BN - 1) / BN;
  const int total_m = __builtin_amdgcn_readfirstlane(sm.tile_start[E]);
  const int total = total_m * n_tiles;
  // each tile's expert by one LDS read instead of a binary search
  const int16_t* mt_tab = total_m <= kMtCap ? sm.mt_expert : nullptr;
  if (mt_tab) {
    for (int tm = tid; tm < total_m; tm += kThreads) sm.mt_expert[tm] = (int16_t)expert_of(tm, sm.tile_start, E);
    __syncthreads();
  }
  // XCD-contiguous tile ranges when the grid is a multiple of 8 workgroups
  // (workgroups go to the XCDs round-robin); the range's workgroups take its
  // tiles in turn
  int begin, end, step, r_lo, j;   // j: this workgroup's index in its range [r_lo, end)
  if ((gridDim.x & 7) == 0) {
    const int per = (total + 7) / 8;
    const int xcd = blockIdx.x & 7;
    j = (int)(blockIdx.x >> 3);
    r_lo = xcd * per;
    begin = r_lo + j;
    end = min(total, (xcd + 1) * per);
    step = gridDim.x >> 3;
  } else {
    j = blockIdx.x;
    r_lo = 0;
    begin = blockIdx.x;
    end = total;
    step = gridDim.x;
  }
  // With QT (the host's choice for dense, one-group launches), a last round
  // that would keep at most a quarter of the range's workgroups busy is split
  // into column quarters, one per workgroup (128 x 128: the
  // wavefronts' weight decodes and MFMAs shrink with the columns, and every
  // output element is formed by the same MFMAs in the same order as in a whole
  // tile).  Quarters have tile indices past the whole tiles.
  int split = end, quarter = kNoTile;
  if constexpr (kQuarters) {
    const int rem = end > r_lo ? (end - r_lo) % step : 0;
    if (rem > 0 && 4 * rem <= step && total <= (0x7fffffff - 8) / 5) {   // quarter indices stay in int
      split = end - rem;
      if ((j >> 2) < rem) quarter = total + 4 * (split + (j >> 2)) + (j & 3);
    }
  }
  // this workgroup's tiles: begin, begin + step, ... below split, then its quarter
  auto next_tile = [&](int L) __attribute__((always_inline)) -> int {
    if constexpr (kQuarters) {
      if (L >= total) return kNoTile;
      return L + step < split ? L + step : quarter;
    } else {
      return L + step < end ? L + step : kNoTile;
    }
  };
  const int first = begin < split ? begin : quarter;
  if (first == kNoTile) return;

  const uint32_t kb = (uint32_t)K / 2, ks = (uint32_t)K / 16;
  const int nk = K / BK;
  // row-major weights: instructions q = wave + kWaves * u of each kind fall to
  // this wavefront
  const int n_loads = KT ? 3 : (kCI - wave + kWaves - 1) / kWaves + (kSI - wave + kWaves - 1) / kWaves;

  // ---------------------------------------------------------------- loads
  // Load cursor: the next K-step to load is (ltile, lk).  Each lane's sources
  // are 32-bit byte offsets from the operand bases (the host keeps every
  // operand under 4 GiB).  A wavefront instruction fills 1 KiB of LDS: 32 code
  // rows or 64 scale dwords.  Activation rows: lane l -> row l/2, 16-byte half
  // l%2 (row-major).  Weight rows: lane l -> row l%32, half l/32, so that a
  // fragment read (16 lanes: 16 rows, one half) covers 256 contiguous bytes.
  int lL = first, lk = 0, nkl = nk;   // the loaded tile's K-steps
  uint32_t off_c[kCIW], off_s[kSIW];
  // Weight K-step strides: row-major [E][N][K/2] moves 32 code bytes (4 scale
  // bytes) along a row per K-step; the K-tiled layout [E][K/64][N][32] moves
  // one whole slab of N rows, and a slab of 32 consecutive rows is 1 KiB of
  // contiguous memory.
  const uint32_t wstep_c = w_tiled ? (uint32_t)N * kRowB : (uint32_t)kRowB;
  const uint32_t wstep_s = w_tiled ? (uint32_t)N * kScB : (uint32_t)kScB;
  // K-tiled weights: three loads per wavefront and K-step.  Slots 0 and 1
  // carry code rows q = w and q = w + 8 (32 rows each; q < 4 are activation
  // rows, the rest weight rows); slot 2 carries code rows q = w + 16 (w < 4),
  // the weight block scales of 256 rows (w = 4, 5: 16 bytes = 4 rows per lane)
  // or the activation block scales of 64 rows (w = 6, 7: 4 bytes per lane).
  // Per slot: the source operand, the per-lane offset of the tile (set per
  // tile), the offset step per K-step and the LDS offset in a stage.
  const uint8_t* src0 = wave < 4 ? a_codes : w_codes;
  const uint8_t* src2 = wave < 4 ? w_codes : wave < 6 ? w_bscales : a_bscales;
  const uint32_t step0 = wave < 4 ? (uint32_t)kRowB : (uint32_t)N * kRowB;
  const uint32_t step1 = (uint32_t)N * kRowB;
  const uint32_t step2 = wave < 4 ? (uint32_t)N * kRowB : wave < 6 ? (uint32_t)N * kScB : (uint32_t)kScB;
  const uint32_t lds_st = (uint32_t)(uintptr_t)(lds_void*)&sm.st[0];
  const uint32_t ldo0 = (uint32_t)wave * 1024u, ldo1 = (uint32_t)(wave + 8) * 1024u;
  const uint32_t ldo2 = wave < 4 ? (uint32_t)(wave + 16) * 1024u
                        : wave < 6 ? (uint32_t)offsetof(Stage, ws) + (uint32_t)(wave - 4) * 1024u
                                   : (uint32_t)offsetof(Stage, as) + (uint32_t)(wave - 6) * 256u;
  uint32_t vo0 = 0, vo1 = 0, vo2 = 0;
  // weight row of stage column c (callers pass c with c % 4 == 0 or a whole
  // 32-column group, so 4 consecutive columns map to 4 consecutive rows);
  // plain tiles: row n0 + c, kept inside the weight matrix by `cap`.  A
  // quarter tile puts its column group g at the stage's 32-column groups 2g
  // and 2g + 8, where wavefronts g and g + 4 find it as their fragment 0 (the
  // odd groups repeat it and are not used).
  auto wcol = [&](const Tile& t, int c, int cap) __attribute__((always_inline)) -> int {
    if constexpr (SW) return ((c >> 5) & 1) * I + (t.n0 >> 1) + ((c >> 6) << 5) + (c & 31);
    else if constexpr (kQuarters) return min(t.n0 + (t.q >= 0 ? ((c >> 1) & 96) + (c & 31) : c), cap);
    else return min(t.n0 + c, cap);
  };
  auto set_load_tile = [&](int L) __attribute__((always_inline)) {
    const Tile t = tile_at<KG, kQuarters>(L, total, n_tiles, sm.tile_start, mt_tab, E, offsets, Mg, kofs, nk);
    nkl = t.nk;
    if constexpr (KT) {
      const int m_last = t.m0 + t.rows - 1;
      const uint32_t half16 = (lane & 1) * 16;
      // K-grouped: activation rows are the group's local rows, and both
      // operands start at the group's first K-step
      const int a_row0 = KG ? t.e * Mg : 0;
      const uint32_t a_k0 = (uint32_t)t.kb0 * kRowB, as_k0 = (uint32_t)t.kb0 * kScB;
      const uint32_t wbase = KG ? (uint32_t)t.kb0 * N : (uint32_t)t.e * nk * N;
      auto wrow = [&](int q) __attribute__((always_inline)) {
        const uint32_t n = (uint32_t)wcol(t, 32 * (q - BM / 32) + (lane & 31), N - 1);
        return (wbase + n) * kRowB + (lane >> 5) * 16;
      };
      vo0 = wave < 4 ? (uint32_t)(min(t.m0 + 32 * wave + (lane >> 1), m_last) - a_row0) * kb + a_k0 + half16
                     : wrow(wave);
      vo1 = wrow(wave + 8);
      if (wave < 4) vo2 = wrow(wave + 16);
      else if (wave < 6) vo2 = (wbase + (uint32_t)wcol(t, 256 * (wave - 4) + 4 * lane, N - 4)) * kScB;
      else vo2 = (uint32_t)(min(t.m0 + 64 * (wave - 6) + lane, m_last) - a_row0) * ks + as_k0;
      return;
    }
    const int m_last = t.m0 + t.rows - 1;
    const int half = lane & 1;
#pragma unroll
    for (int u = 0; u < kCIW; ++u) {
      const int q = wave + kWaves * u;   // code instruction: 0..3 -> A rows, 4.. -> W rows
      if (q < BM / 32) {
        off_c[u] = (uint32_t)min(t.m0 + 32 * q + (lane >> 1), m_last) * kb + half * 16;
      } else {
        const uint32_t n = (uint32_t)wcol(t, 32 * (q - BM / 32) + (lane & 31), N - 1);
        const uint32_t wh = (lane >> 5) * 16;
        off_c[u] = w_tiled ? ((uint32_t)t.e * nk * N + n) * kRowB + wh
                           : ((uint32_t)t.e * N + n) * kb + wh;
      }
    }
#pragma unroll
    for (int u = 0; u < kSIW; ++u) {
      const int q = wave + kWaves * u;   // scale instruction: 0,1 -> A rows, 2.. -> W rows
      if (q < 2) {
        off_s[u] = (uint32_t)min(t.m0 + 64 * q + lane, m_last) * ks;
      } else {
        const uint32_t n = (uint32_t)wcol(t, 64 * (q - 2) + lane, N - 1);
        off_s[u] = w_tiled ? ((uint32_t)t.e * nk * N + n) * kScB : ((uint32_t)t.e * N + n) * ks;
      }
    }
  };
  // issues the loads of the cursor's K-step into stage S and advances the
  // cursor; returns the number of load instructions this wavefront issued
  auto issue_loads = [&](Stage& S) __attribute__((always_inline)) -> int {
    if (lL == kNoTile) return 0;
    if constexpr (KT) {
      const uint32_t ls = lds_st + (uint32_t)((uintptr_t)(lds_void*)&S - (uintptr_t)(lds_void*)&sm.st[0]);
      lds_dma16_at(src0, (uint32_t)lk * step0 + vo0, ls + ldo0);
      lds_dma16_at(w_codes, (uint32_t)lk * step1 + vo1, ls + ldo1);
      if (wave < 6) lds_dma16_at(src2, (uint32_t)lk * step2 + vo2, ls + ldo2);
      else lds_dma4_at(src2, (uint32_t)lk * step2 + vo2, ls + ldo2);
      if (++lk == nkl) {
        lk = 0;
        lL = next_tile(lL);
        if (lL != kNoTile) set_load_tile(lL);
      }
      return 3;
    }
    const uint32_t ka = (uint32_t)lk * kRowB, kss = (uint32_t)lk * kScB;
    const uint32_t kw = (uint32_t)lk * wstep_c, kws = (uint32_t)lk * wstep_s;
#pragma unroll
    for (int u = 0; u < kCIW; ++u) {
      const int q = wave + kWaves * u;
      if (q < BM / 32) lds_dma16(a_codes, ka + off_c[u], S.a + q * 1024);
      else if (q < kCI) lds_dma16(w_codes, kw + off_c[u], S.a + q * 1024);
    }
#pragma unroll
    for (int u = 0; u < kSIW; ++u) {
      const int q = wave + kWaves * u;
      if (q < 2) lds_dma4(a_bscales, kss + off_s[u], S.as + q * 256);
      else if (q < kSI) lds_dma4(w_bscales, kws + off_s[u], S.as + q * 256);
    }
    if (++lk == nkl) {
      lk = 0;
      lL = next_tile(lL);
      if (lL != kNoTile) set_load_tile(lL);
    }
    return n_loads;
  };

  // ---------------------------------------------------------------- decodes
  // activation decode: thread -> row tid/4, elements [16 (tid%4), +16), i.e.
  // one scale block and 16-byte chunks 2 (tid%4), +1 of the FP16 row
  const int drow = tid >> 2, dq = tid & 3;
  uint2 da;          // raw codes of the next K-step's activation share
  uint32_t dsc;      // its block scale
  auto read_a = [&](const Stage& S) __attribute__((always_inline)) {
    da = *reinterpret_cast<const uint2*>(S.a + drow * kRowB + dq * 8);
    dsc = S.as[drow * kScB + dq];
  };
  auto decode_a = [&](uint8_t* A16) __attribute__((always_inline)) {
    const uint32_t s0 = scale_pair(dsc);
    *reinterpret_cast<half8*>(A16 + a16_off(drow, 2 * dq + 0)) = decode8(da.x, s0);
    *reinterpret_cast<half8*>(A16 + a16_off(drow, 2 * dq + 1)) = decode8(da.y, s0);
  };
  // weight fragments: fragment f of this wavefront = the stage's W rows
  // 64 wave + 32 f + (lane % 32) (for a quarter tile, fragment 0 holds the
  // wavefront's column group and fragment 1 is not used); the lane's 32
  // elements [32h, 32h+32) of the K-step are 16 code bytes (word s = the 8
  // elements of MFMA slice s) and block scales 2h, 2h+1 (slices 0-1 and 2-3)
  uint4 rb[FB];
  uint32_t xb[FB];
  auto read_b = [&](const Stage& S) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      const int row = WN * wave + 32 * f + l32;
      rb[f] = *reinterpret_cast<const uint4*>(S.w + (2 * wave + f) * 1024 + h * 512 + l32 * 16);
      xb[f] = *reinterpret_cast<const uint16_t*>(S.ws + row * kScB + h * 2);
    }
  };
  auto word = [](const uint4& v, int s) __attribute__((always_inline)) {
    return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
  };

  // ---------------------------------------------------------------- prologue
  set_load_tile(first);
  issue_loads(sm.st[0]);
  issue_loads(sm.st[1]);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  read_a(sm.st[0]);
  decode_a(sm.a16[0]);
  read_b(sm.st[0]);
  int n_last = issue_loads(sm.st[2]);   // K-step 2 (or nothing)

  half8 bv[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f) bv[f] = decode8(rb[f].x, scale_pair(xb[f] & 0xFF));

  floatx16 acc[FA][FB];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j) acc[i][j] = floatx16{};

  // ---------------------------------------------------------------- main loop
  int sc = 0, ab = 0;   // stage and decoded-activation buffer of the current K-step

  // One K-step of MFMAs (4 slices of 16) with the decodes of the next K-step
  // interleaved.  A fragments are read one slice ahead.  The next K-step's
  // stage is read and decoded even when there is none: the reads stay inside
  // LDS and what they produce is never used.  FULL: all row fragments hold
  // rows; otherwise fragments at or past fa_eff are skipped.  Q: a quarter
  // tile (the wavefront's rows 64 (wave / 4) .. + 63, weight fragment 0).
  // The next K-step's weight fragments are read and their first slice decoded
  // in full: the layout is the same for both kinds of tile.
  auto mma_step = [&](auto full_tag, int fa_eff, auto q_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool Q = decltype(q_tag)::value;
    constexpr int fa = Q ? 2 : FA, fb = Q ? 1 : FB;
    const int r0 = Q ? 64 * (wave >> 2) : 0;
    const uint8_t* A16 = sm.a16[ab];
    uint8_t* A16n = sm.a16[ab ^ 1];
    const Stage& Sn = sm.st[sc == kStages - 1 ? 0 : sc + 1];
    half8 av[FA], bn[FB];
#pragma unroll
    for (int i = 0; i < fa; ++i)
      av[i] = *reinterpret_cast<const half8*>(A16 + a16_off(r0 + 32 * i + l32, 4 * h));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s == 0) read_a(Sn);
      if (s == 1) decode_a(A16n);
      // B values of the next slice (of the next K-step after slice 3)
      if (s < 3) {
#pragma unroll
        for (int j = 0; j < fb; ++j)
          bn[j] = decode8(word(rb[j], s + 1), scale_pair(s + 1 < 2 ? (xb[j] & 0xFF) : (xb[j] >> 8)));
      }
      if (s == 2) read_b(Sn);
      if (s == 3) {
#pragma unroll
        for (int j = 0; j < FB; ++j) bn[j] = decode8(rb[j].x, scale_pair(xb[j] & 0xFF));
      }
#pragma unroll
      for (int i = 0; i < fa; ++i) {
        const half8 a = av[i];
        if (s < 3) av[i] = *reinterpret_cast<const half8*>(A16 + a16_off(r0 + 32 * i + l32, 4 * h + s + 1));
        if (FULL || i < fa_eff) {
#pragma unroll
          for (int j = 0; j < fb; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[j], a, acc[i][j], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < (s < 3 ? fb : FB); ++j) bv[j] = bn[j];
    }
  };

  // Row scales of a tile for its epilogue, into one of two LDS buffers (tile
  // parity): issued at the top of the tile's last K-step, ahead of that step's
  // loads, so that waiting for the loads counted in n_last also waits for them.
  // The row scales go in four loads: wavefronts 0 and 1 the activation rows
  // (64 per load, 4 bytes per lane), 2 and 3 the weight rows (256 per load,
  // 16 bytes = 4 rows per lane).
  const uint32_t lds_rs = (uint32_t)(uintptr_t)(lds_void*)&sm.rs[0][0];
  const uint32_t lds_rw = (uint32_t)(uintptr_t)(lds_void*)&sm.rw[0][0];
  auto issue_rscales = [&](const Tile& t, int rb) __attribute__((always_inline)) {
    const uint32_t dst = lds_rs + (uint32_t)rb * (BM + BN) * 4u;
    if (wave < 2)
      lds_dma4_at(reinterpret_cast<const uint8_t*>(a_rscales),
                  (uint32_t)min(t.m0 + 64 * wave + lane, t.m0 + t.rows - 1) * 4u, dst + wave * 256u);
    else if (wave < 4)
      lds_dma16_at(reinterpret_cast<const uint8_t*>(w_rscales),
                   ((uint32_t)t.e * N + wcol(t, 256 * (wave - 2) + 4 * lane, N - 4)) * 4u,
                   dst + BM * 4u + (wave - 2) * 1024u);
    else if (SW && wave < 6 && w_rows)   // the router weights of the tile's rows
      lds_dma4_at(reinterpret_cast<const uint8_t*>(w_rows),
                  (uint32_t)min(t.m0 + 64 * (wave - 4) + lane, t.m0 + t.rows - 1) * 4u,
                  lds_rw + (uint32_t)rb * BM * 4u + (wave - 4) * 256u);
  };

  // epilogue: C = (acc * s_A[row]) * s_W[col].  Tile (i, j) of the lane holds
  // row 32i + lane%32, columns 32j + 8q + 4h .. +3 (q = 0..3).  Each 32 x 32
  // tile goes through the wavefront's 4 KiB staging slice (16-byte chunks
  // XOR-swizzled by row) and leaves as four stores of 8 rows x 128 contiguous
  // bytes: whole cache lines.  Rows past the tile's valid rows fall outside the
  // buffer's range and are dropped by the hardware; columns past N get an
  // out-of-range offset.  The accumulators are cleared for the next tile.
  auto epilogue = [&](const Tile& t, int rb) __attribute__((always_inline)) {
    const float* rs_a = sm.rs[rb];
    const float* rs_w = sm.rs[rb] + BM;
    if constexpr (kQuarters) {
      if (t.q >= 0) {
        // a quarter tile: the wavefront's fragments are rows r0 + 32 i (i < 2)
        // and columns c0 .. c0 + 31 of the quarter (the stage's columns
        // 64 wave .., whose row scales sit there too), staged and stored as below
        const int r0 = 64 * (wave >> 2), c0 = 32 * (wave & 3);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<float*>(c) + (int64_t)t.m0 * N, (short)0, t.rows * N * 4, 0x00020000);
        uint8_t* stq = sm.stg[wave];
        const int srow = lane >> 3, sch = lane & 7;
        uint32_t srowN = (uint32_t)(srow * N);
        asm volatile("" : "+v"(srowN));
        float4 swv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          swv[q] = *reinterpret_cast<const float4*>(&rs_w[WN * wave + 8 * q + 4 * h]);
        const int n = t.n0 + c0 + 4 * sch;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float sq = rs_a[r0 + 32 * i + l32];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float4 o;
            o.x = (acc[i][0][4 * q + 0] * sq) * swv[q].x;
            o.y = (acc[i][0][4 * q + 1] * sq) * swv[q].y;
            o.z = (acc[i][0][4 * q + 2] * sq) * swv[q].z;
            o.w = (acc[i][0][4 * q + 3] * sq) * swv[q].w;
            *reinterpret_cast<float4*>(stq + l32 * 128 + (((2 * q + h) ^ (l32 & 7)) << 4)) = o;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 8 * r + srow;
            const float4 v = *reinterpret_cast<const float4*>(stq + row * 128 + ((sch ^ (row & 7)) << 4));
            const uint32_t off =
                n < N ? ((uint32_t)((r0 + 32 * i + 8 * r) * N) + srowN + (uint32_t)n) * 4u : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rq, off, 0, kNonTemporal);
          }
          acc[i][0] = floatx16{};
        }
        return;
      }
    }
    float sa[FA];
#pragma unroll
    for (int i = 0; i < FA; ++i) sa[i] = rs_a[32 * i + l32];
    uint8_t* stg = sm.stg[wave];
    if constexpr (SW) {
      // h = (silu(g) * u) * w per (row, h column); the 32 x 32 tile of h (and,
      // if asked for, those of g and u) leave through the staging slice as in
      // the FP32 path below.
      const float* rw = sm.rw[rb];
      float wr[FA];
#pragma unroll
      for (int i = 0; i < FA; ++i) wr[i] = w_rows ? rw[32 * i + l32] : 1.0f;
      float* h_out = static_cast<float*>(c);
      const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
          h_out + (int64_t)t.m0 * I, (short)0, t.rows * I * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
          gu_out + (int64_t)t.m0 * 2 * I, (short)0, gu_out ? t.rows * 2 * I * 4 : 0, 0x00020000);
      const int srow = lane >> 3, sch = lane & 7;
      uint32_t srowI = (uint32_t)(srow * I);
      asm volatile("" : "+v"(srowI));
      const int hc = (t.n0 >> 1) + 32 * wave + 4 * sch;        // h column of the lane's stores
      float4 sg[4], su[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sg[q] = *reinterpret_cast<const float4*>(&rs_w[WN * wave + 8 * q + 4 * h]);
        su[q] = *reinterpret_cast<const float4*>(&rs_w[WN * wave + 32 + 8 * q + 4 * h]);
      }
      auto put = [&](const float4& o, int q) __attribute__((always_inline)) {
        *reinterpret_cast<float4*>(stg + l32 * 128 + (((2 * q + h) ^ (l32 & 7)) << 4)) = o;
      };
      // staged tile -> rows 32 i + (0..31), columns col0 + (0..31) of a matrix with `width` columns
      auto flush = [&](const __amdgpu_buffer_rsrc_t& rs, int i, uint32_t rowW, uint32_t width, int col)
          __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 8 * r + srow;
          const float4 v = *reinterpret_cast<const float4*>(stg + row * 128 + ((sch ^ (row & 7)) << 4));
          const uint32_t off = ((uint32_t)((32 * i + 8 * r) * width) + rowW + (uint32_t)col) * 4u;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kNonTemporal);
        }
      };
#pragma unroll
      for (int i = 0; i < FA; ++i) {
        float4 g[4], u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          g[q].x = (acc[i][0][4 * q + 0] * sa[i]) * sg[q].x;
          g[q].y = (acc[i][0][4 * q + 1] * sa[i]) * sg[q].y;
          g[q].z = (acc[i][0][4 * q + 2] * sa[i]) * sg[q].z;
          g[q].w = (acc[i][0][4 * q + 3] * sa[i]) * sg[q].w;
          u[q].x = (acc[i][1][4 * q + 0] * sa[i]) * su[q].x;
          u[q].y = (acc[i][1][4 * q + 1] * sa[i]) * su[q].y;
          u[q].z = (acc[i][1][4 * q + 2] * sa[i]) * su[q].z;
          u[q].w = (acc[i][1][4 * q + 3] * sa[i]) * su[q].w;
          float4 hv;
          hv.x = swiglu_f32(g[q].x, u[q].x, wr[i]);
          hv.y = swiglu_f32(g[q].y, u[q].y, wr[i]);
          hv.z = swiglu_f32(g[q].z, u[q].z, wr[i]);
          hv.w = swiglu_f32(g[q].w, u[q].w, wr[i]);
          put(hv, q);
        }
        flush(rh, i, srowI, (uint32_t)I, hc);
        if (gu_out) {
#pragma unroll
          for (int q = 0; q < 4; ++q) put(g[q], q);
          flush(rg, i, 2 * srowI, (uint32_t)(2 * I), hc);
#pragma unroll
          for (int q = 0; q < 4; ++q) put(u[q], q);
          flush(rg, i, 2 * srowI, (uint32_t)(2 * I), I + hc);
        }
        acc[i][0] = floatx16{};
        acc[i][1] = floatx16{};
      }
      return;
    }
    constexpr int kOutB = OB ? 2 : 4;             // bytes per output element
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t*>(c) + (int64_t)t.m0 * N * kOutB, (short)0, t.rows * N * kOutB, 0x00020000);
    if constexpr (OB) {
      // BF16: a 32 x 32 tile is 32 rows of 64 bytes; each store instruction
      // writes 16 rows (4 lanes x 16 bytes per row).  Staging: row l32, 8-byte
      // piece 2q + h, the row's four 16-byte chunks XOR-swizzled by row.
      const int srow = lane >> 2, sch = lane & 3;
      uint32_t srowN = (uint32_t)(srow * N);
      asm volatile("" : "+v"(srowN));
#pragma unroll
      for (int j = 0; j < FB; ++j) {
        float4 swv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          swv[q] = *reinterpret_cast<const float4*>(&rs_w[WN * wave + 32 * j + 8 * q + 4 * h]);
        const int n = t.n0 + WN * wave + 32 * j + 8 * sch;
#pragma unroll
        for (int i = 0; i < FA; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float o0 = (acc[i][j][4 * q + 0] * sa[i]) * swv[q].x;
            const float o1 = (acc[i][j][4 * q + 1] * sa[i]) * swv[q].y;
            const float o2 = (acc[i][j][4 * q + 2] * sa[i]) * swv[q].z;
            const float o3 = (acc[i][j][4 * q + 3] * sa[i]) * swv[q].w;
            const uint2 pk = make_uint2(f32_to_bf16_rne(o0) | (f32_to_bf16_rne(o1) << 16),
                                        f32_to_bf16_rne(o2) | (f32_to_bf16_rne(o3) << 16));
            *reinterpret_cast<uint2*>(stg + l32 * 64 + ((q ^ (l32 & 3)) << 4) + 8 * h) = pk;
          }
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int row = 16 * r + srow;
            const uint4 v = *reinterpret_cast<const uint4*>(stg + row * 64 + ((sch ^ (row & 3)) << 4));
            const uint32_t off = n < N ? ((uint32_t)((32 * i + 16 * r) * N) + srowN + (uint32_t)n) * 2u : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc, off, 0, kNonTemporal);
          }
          acc[i][j] = floatx16{};
        }
      }
      return;
    }
    const int srow = lane >> 3, sch = lane & 7;   // store layout: 8 rows x 8 chunks per instruction
    // the lane's row offset, recomputed per tile: kept opaque so that the
    // compiler does not hoist sixteen per-lane row offsets out of the tile loop
    uint32_t srowN = (uint32_t)(srow * N);
    asm volatile("" : "+v"(srowN));
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      float4 swv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        swv[q] = *reinterpret_cast<const float4*>(&rs_w[WN * wave + 32 * j + 8 * q + 4 * h]);
      const int n = t.n0 + WN * wave + 32 * j + 4 * sch;
#pragma unroll
      for (int i = 0; i < FA; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float4 o;
          o.x = (acc[i][j][4 * q + 0] * sa[i]) * swv[q].x;
          o.y = (acc[i][j][4 * q + 1] * sa[i]) * swv[q].y;
          o.z = (acc[i][j][4 * q + 2] * sa[i]) * swv[q].z;
          o.w = (acc[i][j][4 * q + 3] * sa[i]) * swv[q].w;
          *reinterpret_cast<float4*>(stg + l32 * 128 + (((2 * q + h) ^ (l32 & 7)) << 4)) = o;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 8 * r + srow;
          const float4 v = *reinterpret_cast<const float4*>(stg + row * 128 + ((sch ^ (row & 7)) << 4));
          const uint32_t off = n < N ? ((uint32_t)((32 * i + 8 * r) * N) + srowN + (uint32_t)n) * 4u : kOutOfRange;
          // non-temporal: the output is streamed out, not kept in L2 over the tiles' operands
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc, off, 0, kNonTemporal);
        }
        acc[i][j] = floatx16{};
      }
    }
  };

  // The K-steps of one tile.  At the top of each: this wavefront's loads of
  // the next K-step have landed (those of the one after may still be in
  // flight); the barrier publishes everyone's, and the decoded activations of
  // this K-step, and frees the stage that the new loads go to.  The previous
  // tile's epilogue runs after the first of these barriers, so that its stores
  // are issued after every load that this wait has to see complete (vmcnt
  // cannot single out loads that are older than pending stores); its row
  // scales landed with the loads it waited for, and the tile's own row scales
  // go to the other buffer.
  int rbuf = 0;
  auto run_tile = [&](auto full_tag, int fa_eff, const Tile& t, auto q_tag) __attribute__((always_inline)) {
    mma_step(full_tag, fa_eff, q_tag);   // K-step 0: its wait, barrier and loads are done by the caller
    sc = sc == kStages - 1 ? 0 : sc + 1;
    ab ^= 1;
    for (int kt = 1; kt < t.nk; ++kt) {
      wait_vmcnt(n_last);
      lds_barrier();
      if (kt == t.nk - 1) issue_rscales(t, rbuf);
      n_last = issue_loads(sm.st[sc]);
      mma_step(full_tag, fa_eff, q_tag);
      sc = sc == kStages - 1 ? 0 : sc + 1;
      ab ^= 1;
    }
  };

  Tile prev{0, 0, 0, 0, 0, 0, -1};
  for (int L = first; L != kNoTile; L = next_tile(L)) {
    const Tile t = tile_at<KG, kQuarters>(L, total, n_tiles, sm.tile_start, mt_tab, E, offsets, Mg, kofs, nk);
    wait_vmcnt(n_last);
    lds_barrier();
    epilogue(prev, rbuf ^ 1);   // before the first tile: no rows, every store is dropped
    if (t.nk == 1) issue_rscales(t, rbuf);
    n_last = issue_loads(sm.st[sc]);
    bool done = false;
    if constexpr (kQuarters) {
      if (t.q >= 0) {   // the wavefront's rows of a quarter: 64 (wave / 4) .. + 63
        const int fq = min(2, max(0, (t.rows - 64 * (wave >> 2) + 31) >> 5));
        if (fq == 2) run_tile(std::true_type{}, 2, t, std::true_type{});
        else run_tile(std::false_type{}, fq, t, std::true_type{});
        done = true;
      }
    }
    if (!done) {
      const int fa_eff = (t.rows + 31) >> 5;
      if (fa_eff == FA) run_tile(std::true_type{}, FA, t, std::false_type{});
      else run_tile(std::false_type{}, fa_eff, t, std::false_type{});
    }
    prev = t;
    rbuf ^= 1;
  }
  wait_vmcnt(0);    // the last tile's row scales (no loads are left)
  lds_barrier();
  epilogue(prev, rbuf ^ 1);
}

}  // namespace g5
}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" NVFP4MOE_API int nvfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_bscales,
                                               const float* a_rscales,
                                               const int32_t* expert_offsets, int32_t E,
                                               int64_t R_cap, const uint8_t* w_codes,
                                               const uint8_t* w_bscales, const float* w_rscales,
                                               int64_t N, int64_t K, int32_t w_layout, void* c,
                                               int32_t c_dtype, void* stream) {
  if (w_layout != NVFP4_W_ROWMAJOR && w_layout != NVFP4_W_KTILED) return NVFP4_ERR_ARG;
  if (c_dtype != NVFP4_OUT_F32 && c_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_ARG;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS || R_cap < 0) return NVFP4_ERR_SHAPE;
  if (K <= 0 || K % g5::BK != 0 || K > 65536 || N < 16 || N % 16 != 0 || N > (1 << 20))
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
  const int64_t n_tiles = (N + g5::BN - 1) / g5::BN;
  const int64_t max_tiles = ((R_cap + g5::BM - 1) / g5::BM + E) * n_tiles;
  if (max_tiles > INT32_MAX) return NVFP4_ERR_SHAPE;
  // persistent grid: one workgroup per CU on a 256-CU device, a multiple of 8
  int64_t grid = max_tiles < 256 ? max_tiles : 256;
  if (grid >= 8) grid &= ~7ll;
  hipStream_t s = static_cast<hipStream_t>(stream);
#define GG_LAUNCH(KT, OB, QT)                                                                    \
  g5::grouped_gemm_kernel<KT, OB, false, false, QT><<<(unsigned)grid, g5::kThreads, 0, s>>>(  \
      a_codes, a_bscales, a_rscales, expert_offsets, E, w_codes, w_bscales, w_rscales, (int)N, \
      (int)K, c, nullptr, nullptr, 0, nullptr, (int)R_cap)
  // quarter tiles for a sparse last round: dense (one-group) FP32 launches
  const bool kt = w_layout == NVFP4_W_KTILED, ob = c_dtype == NVFP4_OUT_BF16, qt = E == 1;
  if (kt && !ob && qt) GG_LAUNCH(true, false, true);
  else if (kt && !ob) GG_LAUNCH(true, false, false);
  else if (kt) GG_LAUNCH(true, true, false);
  else if (!ob && qt) GG_LAUNCH(false, false, true);
  else if (!ob) GG_LAUNCH(false, false, false);
  else GG_LAUNCH(false, true, false);
#undef GG_LAUNCH
  return launch_status();
}

namespace nvfp4moe {
// w_rows[r] = topk_w[row_to_tk[r]] for the routed rows (the router weight of
// each row of the expert-grouped buffer); a map entry outside [0, R_cap) gives 0
__global__ __launch_bounds__(256) void gather_row_weights_kernel(
    const float* __restrict__ topk_w, const int32_t* __restrict__ row_to_tk,
    const int32_t* __restrict__ offsets, int E, int64_t R_cap, float* __restrict__ w_rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= min((int64_t)offsets[E], R_cap)) return;
  const int32_t i = row_to_tk[r];
  w_rows[r] = (i >= 0 && i < R_cap) ? topk_w[i] : 0.0f;
}
}  // namespace nvfp4moe

extern "C" NVFP4MOE_API int nvfp4_grouped_gemm_swiglu(
    const uint8_t* a_codes, const uint8_t* a_bscales, const float* a_rscales,
    const int32_t* expert_offsets, int32_t E, int64_t R_cap, const uint8_t* w_codes,
    const uint8_t* w_bscales, const float* w_rscales, int64_t I, int64_t K, const float* topk_w,
    const int32_t* row_to_tk, float* h, float* gu, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS || R_cap < 0) return NVFP4_ERR_SHAPE;
  if (K <= 0 || K % g5::BK != 0 || K > 65536) return NVFP4_ERR_SHAPE;
  if (I < g5::BN / 2 || I % (g5::BN / 2) != 0 || 2 * I > (1 << 20)) return NVFP4_ERR_SHAPE;
  if (R_cap > INT32_MAX / 2 || (int64_t)E * 2 * I > INT32_MAX) return NVFP4_ERR_SHAPE;
  if (R_cap * (K / 2) > (int64_t)UINT32_MAX || (int64_t)E * 2 * I * (K / 2) > (int64_t)UINT32_MAX)
    return NVFP4_ERR_SHAPE;
  if (R_cap == 0) return NVFP4_OK;
  if (!a_codes || !a_bscales || !a_rscales || !expert_offsets || !w_codes || !w_bscales ||
      !w_rscales || !h)
    return NVFP4_ERR_NULL;
  if (topk_w && (!row_to_tk || !workspace)) return NVFP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_bscales) || !aligned16(a_rscales) ||
      !aligned16(w_codes) || !aligned16(w_bscales) || !aligned16(w_rscales) || !aligned16(h) ||
      !aligned16(gu) || !aligned16(workspace))
    return NVFP4_ERR_ALIGN;
  if (topk_w && workspace_bytes < (size_t)R_cap * sizeof(float)) return NVFP4_ERR_WORKSPACE;
  const int64_t n_tiles = I / (g5::BN / 2);
  const int64_t max_tiles = ((R_cap + g5::BM - 1) / g5::BM + E) * n_tiles;
  if (max_tiles > INT32_MAX) return NVFP4_ERR_SHAPE;
  int64_t grid = max_tiles < 256 ? max_tiles : 256;
  if (grid >= 8) grid &= ~7ll;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* w_rows = nullptr;
  if (topk_w) {
    w_rows = static_cast<float*>(workspace);
    gather_row_weights_kernel<<<(unsigned)((R_cap + 255) / 256), 256, 0, s>>>(
        topk_w, row_to_tk, expert_offsets, E, R_cap, w_rows);
  }
  g5::grouped_gemm_kernel<true, false, true, false><<<(unsigned)grid, g5::kThreads, 0, s>>>(
      a_codes, a_bscales, a_rscales, expert_offsets, E, w_codes, w_bscales, w_rscales,
      (int)(2 * I), (int)K, h, w_rows, gu, (int)I, nullptr, (int)R_cap);
  return launch_status();
}

extern "C" NVFP4MOE_API int nvfp4_grouped_gemm_wgrad(
    const uint8_t* a_codes, const uint8_t* a_bscales, const float* a_rscales,
    const uint8_t* w_codes, const uint8_t* w_bscales, const float* w_rscales,
    const int32_t* kofs, int32_t E, int64_t M, int64_t N, int64_t Kp, void* c, int32_t c_dtype,
    void* stream) {
  if (c_dtype != NVFP4_OUT_F32 && c_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_ARG;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS || M < 1 || N < 16 || N % 16 != 0 || N > (1 << 20))
    return NVFP4_ERR_SHAPE;
  if (Kp <= 0 || Kp % g5::BK != 0) return NVFP4_ERR_SHAPE;
  if ((int64_t)E * M > INT32_MAX / 2 || (int64_t)E * N > INT32_MAX) return NVFP4_ERR_SHAPE;
  // 32-bit byte offsets into each operand
  if (M * (Kp / 2) > (int64_t)UINT32_MAX || N * (Kp / 2) > (int64_t)UINT32_MAX) return NVFP4_ERR_SHAPE;
  if (!a_codes || !a_bscales || !a_rscales || !w_codes || !w_bscales || !w_rscales || !kofs || !c)
    return NVFP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_bscales) || !aligned16(a_rscales) ||
      !aligned16(w_codes) || !aligned16(w_bscales) || !aligned16(w_rscales) || !aligned16(c))
    return NVFP4_ERR_ALIGN;
  const int64_t max_tiles = (int64_t)E * ((M + g5::BM - 1) / g5::BM) * ((N + g5::BN - 1) / g5::BN);
  if (max_tiles > INT32_MAX) return NVFP4_ERR_SHAPE;
  int64_t grid = max_tiles < 256 ? max_tiles : 256;
  if (grid >= 8) grid &= ~7ll;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c_dtype == NVFP4_OUT_BF16)
    g5::grouped_gemm_kernel<true, true, false, true><<<(unsigned)grid, g5::kThreads, 0, s>>>(
        a_codes, a_bscales, a_rscales, nullptr, E, w_codes, w_bscales, w_rscales, (int)N, (int)Kp, c,
        nullptr, nullptr, 0, kofs, (int)M);
  else
    g5::grouped_gemm_kernel<true, false, false, true><<<(unsigned)grid, g5::kThreads, 0, s>>>(
        a_codes, a_bscales, a_rscales, nullptr, E, w_codes, w_bscales, w_rscales, (int)N, (int)Kp, c,
        nullptr, nullptr, 0, kofs, (int)M);
  return launch_status();
}
