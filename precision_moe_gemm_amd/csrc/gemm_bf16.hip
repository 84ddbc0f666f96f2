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
// The two dgrad GEMMs of a MoE layer read 0.4 and 0.8 GB of BF16 weights, so
// they are bound by memory, not by the matrix cores; the design keeps many
// bytes in flight and reads every byte from L2 as few times as it can:
//   * one 512-thread workgroup per CU, tile 256 rows x 256 columns (8
//     wavefronts of 128 x 64), K-step 32;
//   * A rows and weight rows go from global memory straight into LDS
//     (global_load_lds) in a 4-stage ring, three K-steps ahead; the load
//     cursor runs on into the next tile, so the ring never drains;
//   * the MFMA (v_mfma_f32_16x16x32_bf16) computes C^T tiles, weights as its
//     first operand, which leaves 4 consecutive output columns in each lane for
//     16-byte stores.  The activation tile's 16-byte chunks are XOR-swizzled by
//     row (conflict-free fragment reads); a [K][N] weight tile keeps its rows
//     in LDS (16-byte chunks XOR-swizzled by row) and each fragment is read
//     with two transposing LDS reads (ds_read_b64_tr_b16);
//   * a tile's stores are issued after the first barrier of the next tile, so
//     a wait for loads never has to cover them;
//   * tiles are scheduled like the NVFP4 GEMM: persistent workgroups,
//     XCD-contiguous ranges, m-tile major, expert rows from device offsets;
//     row fragments past an expert's end are skipped.
#include "common.h"

#include <type_traits>

namespace nvfp4moe {
namespace gb {

// Tile BM x 256 (BM = 2 * WM: 256, or 128 when the grid would otherwise get
// too few tiles), 8 wavefronts of WM x 64.
constexpr int BN = 256, BK = 32;
constexpr int kWaves = 8, kThreads = kWaves * 64;
constexpr int kLdsStages = 147456;            // LDS for the stage ring (144 KiB)
constexpr int kRowB = BK * 2;                 // 64 bytes of a row per K-step
constexpr int WN = 64, FN = WN / 16;          // wavefront columns: 4 MFMA 16x16 tiles
constexpr int kWI = BN * kRowB / 1024 / kWaves;   // weight load instructions per wavefront per K-step (2)
constexpr int kMaxBM = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// A stage: the activation tile, [BM rows][4 chunks of 16 B] with chunks
// XOR-swizzled by row, then the weight tile, [32 k][256 n] (KN) or like the
// activations (NK).  As many stages as fit kLdsStages: 4 for BM = 256, 6 for
// BM = 128.
struct Stage {
  uint8_t* a;
  uint8_t* w;
};

struct __align__(16) Smem {
  uint8_t ring[kLdsStages];
  int tile_start[NVFP4MOE_MAX_EXPERTS + 1];
};

// physical 16-byte chunk of logical chunk c (0..3) of row r: rows r..r+15 of
// one fragment read land in 16 distinct 16-byte bank groups
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Direct-to-LDS load: each lane's 16 bytes at base + voff land at lds + 16 * lane.
// Issued through inline assembly so that the compiler does not make every
// later LDS read wait for it; the kernel waits itself (vmcnt).
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, const uint8_t* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt vmcnt(n), n in [0, 15], with expcnt and lgkmcnt at their maxima
  switch (n) {
#define GB_W(i) case i: __builtin_amdgcn_s_waitcnt(0x0F70 | i); break;
    GB_W(1) GB_W(2) GB_W(3) GB_W(4) GB_W(5) GB_W(6) GB_W(7) GB_W(8) GB_W(9) GB_W(10) GB_W(11)
    GB_W(12) GB_W(13) GB_W(14) GB_W(15)
#undef GB_W
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

struct Tile {
  int e, m0, rows, n0;
};

template <int BM>
__device__ __forceinline__ Tile tile_at(int L, int n_tiles, const int* tile_start, int E,
                                        const int32_t* __restrict__ offsets) {
  const int tm = L / n_tiles, tn = L - tm * n_tiles;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= tm) lo = mid; else hi = mid;
  }
  Tile t;
  t.e = __builtin_amdgcn_readfirstlane(lo);
  t.m0 = __builtin_amdgcn_readfirstlane(offsets[t.e] + (tm - tile_start[t.e]) * BM);
  t.rows = __builtin_amdgcn_readfirstlane(min(BM, offsets[t.e + 1] - t.m0));
  t.n0 = tn * BN;
  return t;
}

template <bool KN, int WM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bf16_grouped_gemm_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ offsets,
                              int E, const uint16_t* __restrict__ w, int N, int K,
                              float* __restrict__ c) {
  constexpr int BM = 2 * WM, FM = WM / 16;
  constexpr int kAI = BM * kRowB / 1024 / kWaves;   // A load instructions per wavefront per K-step
  constexpr int kStageB = (BM + BN) * kRowB;
  constexpr int kStages = kLdsStages / kStageB;
  static_assert(kStages >= 3 && (kStages - 2) * (kAI + kWI) <= 15, "stage ring");
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
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
      if (e < E) sm.tile_start[e] = carry + incl - v;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) sm.tile_start[E] = carry;
  }
  __syncthreads();

  const int n_tiles = (N + BN - 1) / BN;
  const int total = __builtin_amdgcn_readfirstlane(sm.tile_start[E]) * n_tiles;
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
  if (begin >= end) return;
  const int nk = K / BK;

  // ------------------------------------------------------------ load cursor
  // (lL, lk): the next K-step to load.  Each lane's sources are 32-bit byte
  // offsets from the operand bases (the host keeps both under 4 GiB).  Instruction q
  // of an operand fills 1 KiB: A (and NK weight) rows 16q .. 16q+15, lane l ->
  // row 16q + l/4, physical chunk l%4; KN weight rows k = 2q, 2q+1, lane l ->
  // k = 2q + l/32, columns 8 (l%32) .. +7.
  int lL = begin, lk = 0;
  uint32_t off_a[kAI], off_w[kWI];
  auto set_load_tile = [&](int L) __attribute__((always_inline)) {
    const Tile t = tile_at<BM>(L, n_tiles, sm.tile_start, E, offsets);
#pragma unroll
    for (int u = 0; u < kAI; ++u) {
      const int q = wave * kAI + u;
      const int r = 16 * q + (lane >> 2);
      const int m = min(t.m0 + r, t.m0 + t.rows - 1);
      off_a[u] = ((uint32_t)m * K + 8 * swz(r, lane & 3)) * 2u;
    }
#pragma unroll
    for (int u = 0; u < kWI; ++u) {
      const int q = wave * kWI + u;
      if (KN) {
        // physical chunk lane%32 of row k holds logical chunk (lane%32) ^ 2(k%4)
        const int k = 2 * q + (lane >> 5);
        const int n = min(t.n0 + 8 * ((lane & 31) ^ (2 * (k & 3))), N - 8);
        off_w[u] = (((uint32_t)t.e * K + k) * N + n) * 2u;
      } else {
        const int r = 16 * q + (lane >> 2);
        const int n = min(t.n0 + r, N - 1);
        off_w[u] = (((uint32_t)t.e * N + n) * K + 8 * swz(r, lane & 3)) * 2u;
      }
    }
  };
  // loads of the cursor's K-step into stage S; returns the instructions issued
  auto stage = [&](int i) __attribute__((always_inline)) -> Stage {
    return Stage{sm.ring + i * kStageB, sm.ring + i * kStageB + BM * kRowB};
  };
  auto issue_loads = [&](const Stage& S) __attribute__((always_inline)) -> int {
    if (lL >= end) return 0;
    const uint32_t ka = (uint32_t)lk * kRowB;
    const uint32_t kw = KN ? (uint32_t)lk * BK * N * 2u : (uint32_t)lk * kRowB;
#pragma unroll
    for (int u = 0; u < kAI; ++u) lds_dma16(a, off_a[u] + ka, S.a + (wave * kAI + u) * 1024);
#pragma unroll
    for (int u = 0; u < kWI; ++u) lds_dma16(w, off_w[u] + kw, S.w + (wave * kWI + u) * 1024);
    if (++lk == nk) {
      lk = 0;
      lL += step;
      if (lL < end) set_load_tile(lL);
    }
    return kAI + kWI;
  };

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // one K-step of MFMAs from stage S; FULL: every row fragment holds rows
  auto mma_step = [&](auto full_tag, int fm_eff, const Stage& S) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    bf16x8 bv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = WN * wn + 16 * j + l16;
      if (KN) {
        // Transposing reads (ds_read_b64_tr_b16): in each group of 16 lanes,
        // lane p points at columns 4(p%4)..+3 of row k0 + p/4 of the
        // fragment's 16 columns, and lane i receives column i of rows
        // k0..k0+3.  Two reads give the 8 K values of the lane's column.
        const int col = WN * wn + 16 * j + 4 * (l16 & 3);
        v4i16 v[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = 8 * g + 4 * hh + (l16 >> 2);
          const int pc = (col >> 3) ^ (2 * (k & 3));
          v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(S.w + k * (BN * 2) + pc * 16 + ((col >> 2) & 1) * 8));
        }
        bv[j] = __builtin_bit_cast(bf16x8, (v8i16){v[0][0], v[0][1], v[0][2], v[0][3],
                                                   v[1][0], v[1][1], v[1][2], v[1][3]});
      } else {
        bv[j] = *reinterpret_cast<const bf16x8*>(S.w + n * kRowB + swz(n, g) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (FULL || i < fm_eff) {
        const int r = WM * wm + 16 * i + l16;
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(S.a + r * kRowB + swz(r, g) * 16);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[j], av, acc[i][j], 0, 0, 0);
      }
    }
  };

  // C = acc^T: lane (l16, g) of tile (i, j) holds row 16i + l16, columns
  // 16j + 4g .. +3 of the wavefront's block; rows past the tile's rows and
  // columns past N are not written.  The accumulators are cleared.
  auto epilogue = [&](const Tile& t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = WM * wm + 16 * i + l16;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = t.n0 + WN * wn + 16 * j + 4 * g;
        if (r < t.rows && n < N)
          *reinterpret_cast<floatx4*>(c + (int64_t)(t.m0 + r) * N + n) = acc[i][j];
        acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  // ------------------------------------------------------------ pipeline
  // At the top of K-step g: this wavefront's loads of g have landed (those of
  // g+1 and g+2 may be in flight); the barrier publishes everyone's and frees
  // the stage of g-1, which the loads of g+3 then fill.
  // nq[i]: this wavefront's load instructions of K-step g + i (g: the next
  // K-step to compute), for the kStages - 1 K-steps in flight
  set_load_tile(begin);
  int nq[kStages - 1];
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i) nq[i] = issue_loads(stage(i));
  int sc = 0;
  auto top = [&]() __attribute__((always_inline)) {
    int later = 0;
#pragma unroll
    for (int i = 1; i < kStages - 1; ++i) later += nq[i];
    wait_vmcnt(later);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kStages - 2; ++i) nq[i] = nq[i + 1];
    nq[kStages - 2] = issue_loads(stage(sc == 0 ? kStages - 1 : sc - 1));
  };
  auto run_tile = [&](auto full_tag, int fm_eff) __attribute__((always_inline)) {
    mma_step(full_tag, fm_eff, stage(sc));   // K-step 0: its top is done by the caller
    sc = sc == kStages - 1 ? 0 : sc + 1;
    for (int kt = 1; kt < nk; ++kt) {
      top();
      mma_step(full_tag, fm_eff, stage(sc));
      sc = sc == kStages - 1 ? 0 : sc + 1;
    }
  };

  Tile prev{0, 0, 0, 0};
  for (int L = begin; L < end; L += step) {
    const Tile t = tile_at<BM>(L, n_tiles, sm.tile_start, E, offsets);
    top();
    epilogue(prev);   // before the first tile: no rows, nothing is written
    const int fm_eff = min(FM, max(0, (t.rows - WM * wm + 15) >> 4));
    if (t.rows == BM) run_tile(std::true_type{}, FM);
    else run_tile(std::false_type{}, fm_eff);
    prev = t;
  }
  epilogue(prev);
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
  // the kernel addresses both operands with 32-bit byte offsets
  if (R_cap * K * 2 > (int64_t)UINT32_MAX || (int64_t)E * N * K * 2 > (int64_t)UINT32_MAX ||
      R_cap > INT32_MAX / 2)
    return NVFP4_ERR_SHAPE;
  if (R_cap == 0) return NVFP4_OK;
  if (!a || !expert_offsets || !w || !c) return NVFP4_ERR_NULL;
  if (!aligned16(a) || !aligned16(w) || !aligned16(c)) return NVFP4_ERR_ALIGN;
  const int64_t n_tiles = (N + gb::BN - 1) / gb::BN;
  // 256-row tiles when the expected tile count (the routing is on the device:
  // about R/BM + E/2 row tiles) keeps the 256 workgroups busy for 4 rounds,
  // else 128-row tiles
  const bool tall = (R_cap / 256 + E / 2) * n_tiles >= 4 * 256;
  const int64_t bm = tall ? 256 : 128;
  const int64_t max_tiles = ((R_cap + bm - 1) / bm + E) * n_tiles;
  if (max_tiles > INT32_MAX) return NVFP4_ERR_SHAPE;
  // persistent grid: one workgroup per CU on a 256-CU device, a multiple of 8
  int64_t grid = max_tiles < 256 ? max_tiles : 256;
  if (grid >= 8) grid &= ~7ll;
  hipStream_t s = static_cast<hipStream_t>(stream);
#define GB_LAUNCH(KN_, WM_)                                                                   \
  gb::bf16_grouped_gemm_kernel<KN_, WM_><<<(unsigned)grid, gb::kThreads, 0, s>>>(             \
      a, expert_offsets, E, w, (int)N, (int)K, c)
  if (w_layout == NVFP4MOE_W_KN) {
    if (tall) GB_LAUNCH(true, 128); else GB_LAUNCH(true, 64);
  } else {
    if (tall) GB_LAUNCH(false, 128); else GB_LAUNCH(false, 64);
  }
#undef GB_LAUNCH
  return launch_status();
}
