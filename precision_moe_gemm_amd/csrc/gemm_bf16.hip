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
//   * one 512-thread workgroup per CU, tiles of up to 320 rows x 256 columns
//     (8 wavefronts of up to 160 x 64; the two wavefront rows take alternate
//     16-row groups), K-step 32.  The tile height (320, 256, 192, 160, 128 or
//     64) is picked per launch from the routing: an expert of up to 320 rows
//     then streams each weight slab once, while a skewed routing gets shorter
//     tiles that spread its large experts over more workgroups; an expert's
//     rows are split evenly over its tiles (in 16-row groups), so that its
//     tiles cost about the same;
//   * the MFMA loop is compiled once per count of 16-row groups a wavefront
//     holds, so a partial tile runs straight-line code with every fragment
//     read issued before its MFMAs;
//   * A rows and weight rows go from global memory straight into LDS
//     (global_load_lds) in a 4-stage ring, three K-steps ahead; the load
//     cursor runs on into the next tile, so the ring never drains;
//   * the MFMA (v_mfma_f32_16x16x32_bf16) computes C^T tiles, weights as its
//     first operand, which leaves 4 consecutive output columns in each lane for
//     16-byte stores.  The activation tile's 16-byte chunks are XOR-swizzled by
//     row (conflict-free fragment reads); a [K][N] weight tile keeps its rows
//     in LDS (16-byte chunks XOR-swizzled by row, wswz) and each fragment is read
//     with two transposing LDS reads (ds_read_b64_tr_b16);
//   * a tile's stores are issued after the first barrier of the next tile, so
//     a wait for loads never has to cover them;
//   * tiles are scheduled like the NVFP4 GEMM: persistent workgroups,
//     XCD-contiguous ranges, m-tile major, expert rows from device offsets;
//     row groups past an expert's end are neither loaded nor multiplied.
#include "common.h"

#include <type_traits>
#include <utility>

namespace nvfp4moe {
namespace gb {

// Tiles of up to BM x 256, 8 wavefronts of up to WM x 64; the tile height
// (kHeights) is chosen per launch from the routing.
constexpr int BM = 320, WM = BM / 2, FM = WM / 16;
constexpr int BN = 256, BK = 32;
constexpr int kNumHeights = 6;
constexpr int kHeights[kNumHeights] = {320, 256, 192, 160, 128, 64};
constexpr int kTileCost = 96;                 // rows' worth of per-tile cost (see the kernel)
constexpr int kWaves = 8, kThreads = kWaves * 64;
constexpr int kLdsStages = 147456;            // LDS for the stage ring (144 KiB)
constexpr int kRowB = BK * 2;                 // 64 bytes of a row per K-step
constexpr int WN = 64, FN = WN / 16;          // wavefront columns: 4 MFMA 16x16 tiles
constexpr int kWI = BN * kRowB / 1024 / kWaves;   // weight load instructions per wavefront per K-step (2)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// A stage: the activation tile, [BM rows][4 chunks of 16 B] with chunks
// XOR-swizzled by row, then the weight tile, [32 k][256 n] (KN) or like the
// activations (NK).  As many stages as fit kLdsStages: 4.
struct Stage {
  uint8_t* a;
  uint8_t* w;
};

struct __align__(16) Smem {
  uint8_t ring[kLdsStages];
  int tile_start[NVFP4MOE_MAX_EXPERTS + 1];
  int bm;
};

// physical 16-byte chunk of logical chunk c (0..3) of row r.  A 16-byte LDS
// read (ds_read_b128) on gfx950 is served in four passes of 16 lanes; a pass
// takes, from one half of the wavefront (lanes 0-31 or 32-63), the four lane
// quads whose quad index (lane / 4) mod 8 has the same bit parity, and is
// conflict-free when its 16 reads fall on the 16 distinct 16-byte bank groups
// of a 256-byte window (measured with SQ_LDS_BANK_CONFLICT on single-pattern
// kernels).  A fragment read gives lane (l, g) row r0 + l (l < 16), chunk g:
// with the XOR below each pass covers rows 4i..4i+3 of two row quads whose
// XOR terms differ, i.e. 16 distinct (row mod 4, chunk) pairs.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 2); }

// [K][N] weight tile: physical 16-byte chunk p of row k holds logical chunk
// p ^ wswz(k).  A transposing read covers rows k0..k0+3 in each group of 16
// lanes, and one LDS cycle serves two groups, whose rows are 8 apart: the
// 2 (k % 4) term spreads the 4 rows over distinct banks, the 8 ((k / 8) % 2)
// term moves the second group's rows to the other half of the banks.
__device__ __forceinline__ int wswz(int k) { return (2 * (k & 3)) | (8 * ((k >> 3) & 1)); }

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

// fn(std::integral_constant<int, v>) for the v in Is... equal to n
template <int... Is, typename Fn>
__device__ __forceinline__ void dispatch_count(int n, std::integer_sequence<int, Is...>, Fn&& fn) {
  (void)((n == Is ? (fn(std::integral_constant<int, Is>{}), true) : false) || ...);
}

struct Tile {
  int e, m0, rows, n0;
};

// expert offsets clamped into [0, Rc] (the rows of the output buffer): malformed
// offsets give wrong rows but no access outside the buffers
__device__ __forceinline__ int off_at(const int32_t* __restrict__ offsets, int Rc, int e) {
  return min(max(offsets[e], 0), Rc);
}

__device__ __forceinline__ Tile tile_at(int L, int n_tiles, int bm, const int* tile_start, int E,
                                        const int32_t* __restrict__ offsets, int Rc) {
  const int tm = L / n_tiles, tn = L - tm * n_tiles;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= tm) lo = mid; else hi = mid;
  }
  Tile t;
  t.e = __builtin_amdgcn_readfirstlane(lo);
  // the expert's rows split evenly over its nt = ceil(rows / bm) m-tiles, in
  // 16-row groups: per <= bm (bm is a multiple of 16), and (nt - 1) * per <
  // rows, so no tile is empty or taller than bm
  const int o0 = off_at(offsets, Rc, t.e), o1 = off_at(offsets, Rc, t.e + 1);
  const int nt = tile_start[t.e + 1] - tile_start[t.e];
  const int per = ((o1 - o0 + nt - 1) / nt + 15) & ~15;
  t.m0 = __builtin_amdgcn_readfirstlane(o0 + (tm - tile_start[t.e]) * per);
  t.rows = __builtin_amdgcn_readfirstlane(max(0, min(per, o1 - t.m0)));
  t.n0 = tn * BN;
  return t;
}

template <bool KN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bf16_grouped_gemm_kernel(const uint16_t* __restrict__ a, const int32_t* __restrict__ a_map,
                              int a_div, int a_rows, const int32_t* __restrict__ offsets,
                              int E, int Rc, const uint16_t* __restrict__ w, int N, int K,
                              float* __restrict__ c) {
  constexpr int kAF = BM / 16;                      // A load instructions per K-step (16 rows each)
  constexpr int kAI = (kAF + kWaves - 1) / kWaves;  // ... per wavefront, at most
  constexpr int kStageB = (BM + BN) * kRowB;
  constexpr int kStages = kLdsStages / kStageB;
  static_assert(kStages >= 3 && (kStages - 2) * (kAI + kWI) <= 15, "stage ring");
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int l16 = lane & 15, g = lane >> 4;

  const int n_tiles = (N + BN - 1) / BN;
  if (wave == 0) {
    // Tile height: the candidate with the smallest estimated critical path,
    // (tiles per workgroup) x (height + kTileCost), the last term standing for
    // a tile's cost that does not scale with its rows (the weight slab it
    // streams).  Taller tiles read each expert's weights fewer times; shorter
    // ones spread a skewed routing over more workgroups.  Ties go to the taller.
    const int G = gridDim.x, xg = (G & 7) == 0 ? 8 : 1;
    int best = kHeights[0];
    int64_t best_cost = INT64_MAX;
#pragma unroll
    for (int c = 0; c < kNumHeights; ++c) {
      const int h = kHeights[c];
      int mt = 0;
      for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        int v = e < E ? max(0, off_at(offsets, Rc, e + 1) - off_at(offsets, Rc, e) + h - 1) / h : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
        mt += v;
      }
      const int64_t total = (int64_t)mt * n_tiles;
      const int64_t per = (total + xg - 1) / xg, wgs = G / xg;
      const int64_t cost = (per + wgs - 1) / wgs * (h + kTileCost);
      if (cost < best_cost) {
        best_cost = cost;
        best = h;
      }
    }
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int v = e < E ? max(0, off_at(offsets, Rc, e + 1) - off_at(offsets, Rc, e) + best - 1) / best : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      if (e < E) sm.tile_start[e] = carry + incl - v;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      sm.tile_start[E] = carry;
      sm.bm = best;
    }
  }
  __syncthreads();

  const int bm = __builtin_amdgcn_readfirstlane(sm.bm);
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
  // k = 2q + l/32, columns 8 (l%32) .. +7.  Wavefront v issues the A
  // instructions q = v, v + 8, ... that hold rows of the tile (none past its
  // last 16-row group) and the weight instructions 2v, 2v + 1.
  int lL = begin, lk = 0;
  uint32_t off_a[kAI], off_w[kWI];
  int na = 0;   // A instructions of this wavefront for the load tile: q = wave + 8u < ceil(rows / 16)
  auto set_load_tile = [&](int L) __attribute__((always_inline)) {
    const Tile t = tile_at(L, n_tiles, bm, sm.tile_start, E, offsets, Rc);
    const int fa = min(kAF, (t.rows + 15) >> 4);
    na = fa > wave ? (fa - wave + kWaves - 1) / kWaves : 0;
#pragma unroll
    for (int u = 0; u < kAI; ++u) {
      const int q = wave + kWaves * u;
      const int r = 16 * q + (lane >> 2);
      int m = min(t.m0 + r, t.m0 + t.rows - 1);
      // gathered operand: routed row m reads row a_map[m] / a_div of a,
      // clamped into a (an invalid map entry reads a wrong row, never outside)
      if (a_map) m = min(max(a_map[m], 0) / a_div, a_rows - 1);
      off_a[u] = ((uint32_t)m * K + 8 * swz(r, lane & 3)) * 2u;
    }
#pragma unroll
    for (int u = 0; u < kWI; ++u) {
      const int q = wave * kWI + u;
      if (KN) {
        // physical chunk lane%32 of row k holds logical chunk (lane%32) ^ 2(k%4)
        const int k = 2 * q + (lane >> 5);
        const int n = min(t.n0 + 8 * ((lane & 31) ^ wswz(k)), N - 8);
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
    for (int u = 0; u < kAI; ++u)
      if (u < na) lds_dma16(a, off_a[u] + ka, S.a + (wave + kWaves * u) * 1024);
#pragma unroll
    for (int u = 0; u < kWI; ++u) lds_dma16(w, off_w[u] + kw, S.w + (wave * kWI + u) * 1024);
    if (++lk == nk) {
      lk = 0;
      lL += step;
      if (lL < end) set_load_tile(lL);
    }
    return na + kWI;
  };

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // one K-step of MFMAs from stage S over the wavefront's first NF row
  // fragments (a compile-time count, so that every variant is straight-line
  // code the compiler can schedule across fragments)
  auto mma_step = [&](auto nf_tag, const Stage& S) __attribute__((always_inline)) {
    constexpr int NF = decltype(nf_tag)::value;
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
          const int pc = (col >> 3) ^ wswz(k);
          v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(S.w + k * (BN * 2) + pc * 16 + ((col >> 2) & 1) * 8));
        }
        bv[j] = __builtin_bit_cast(bf16x8, (v8i16){v[0][0], v[0][1], v[0][2], v[0][3],
                                                   v[1][0], v[1][1], v[1][2], v[1][3]});
      } else {
        bv[j] = *reinterpret_cast<const bf16x8*>(S.w + n * kRowB + swz(n, g) * 16);
      }
    }
    // every fragment read is issued before the first MFMA (kept there by the
    // scheduling barrier), so that the MFMAs wait on reads issued long before
    bf16x8 av[FM];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int r = 32 * i + 16 * wm + l16;
      av[i] = *reinterpret_cast<const bf16x8*>(S.a + r * kRowB + swz(r, g) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[j], av[i], acc[i][j], 0, 0, 0);
  };

  // C = acc^T: lane (l16, g) of tile (i, j) holds tile row 32i + 16wm + l16
  // (the two wavefront rows take alternate 16-row groups, so a partial tile
  // splits evenly), columns 16j + 4g .. +3 of the wavefront's 64; rows past the tile's rows and
  // columns past N are not written.  The accumulators are cleared.
  auto epilogue = [&](const Tile& t) __attribute__((always_inline)) {
    // the lane's position, recomputed here: a value carried from the prologue
    // would hold a register through the K-loop (which has none to spare)
    int le;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(le));
    const int l16e = le & 15, ge = le >> 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = 32 * i + 16 * wm + l16e;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = t.n0 + WN * wn + 16 * j + 4 * ge;
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
  auto run_tile = [&](auto nf_tag) __attribute__((always_inline)) {
    mma_step(nf_tag, stage(sc));   // K-step 0: its top is done by the caller
    sc = sc == kStages - 1 ? 0 : sc + 1;
    for (int kt = 1; kt < nk; ++kt) {
      top();
      mma_step(nf_tag, stage(sc));
      sc = sc == kStages - 1 ? 0 : sc + 1;
    }
  };

  Tile prev{0, 0, 0, 0};
  for (int L = begin; L < end; L += step) {
    const Tile t = tile_at(L, n_tiles, bm, sm.tile_start, E, offsets, Rc);
    top();
    epilogue(prev);   // before the first tile: no rows, nothing is written
    const int fm_eff = min(FM, (((t.rows + 15) >> 4) - wm + 1) >> 1);
    dispatch_count(fm_eff, std::make_integer_sequence<int, FM + 1>{},
                   [&](auto nf_tag) __attribute__((always_inline)) { run_tile(nf_tag); });
    prev = t;
  }
  epilogue(prev);
}

}  // namespace gb
}  // namespace nvfp4moe

using namespace nvfp4moe;

namespace {

int launch_bf16_grouped_gemm(const uint16_t* a, int64_t a_rows, const int32_t* a_map, int32_t a_div,
                             const int32_t* expert_offsets, int32_t E, int64_t R_cap,
                             const uint16_t* w, int32_t w_layout, int64_t N, int64_t K, float* c,
                             void* stream) {
  if (w_layout != NVFP4MOE_W_KN && w_layout != NVFP4MOE_W_NK) return NVFP4_ERR_ARG;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS || R_cap < 0 || a_rows < 0) return NVFP4_ERR_SHAPE;
  if (K <= 0 || K % gb::BK != 0 || N < 16 || N % 16 != 0) return NVFP4_ERR_SHAPE;
  // the kernel addresses both operands with 32-bit byte offsets
  if (a_rows * K * 2 > (int64_t)UINT32_MAX || (int64_t)E * N * K * 2 > (int64_t)UINT32_MAX ||
      R_cap > INT32_MAX / 2)
    return NVFP4_ERR_SHAPE;
  if (R_cap == 0) return NVFP4_OK;
  if (a_rows == 0) return NVFP4_ERR_SHAPE;   // routed rows but nothing to read them from
  if (!a || !expert_offsets || !w || !c) return NVFP4_ERR_NULL;
  if (!aligned16(a) || !aligned16(w) || !aligned16(c)) return NVFP4_ERR_ALIGN;
  const int64_t n_tiles = (N + gb::BN - 1) / gb::BN;
  // the most tiles any tile height can give (the kernel picks the height from
  // the routing, which is on the device)
  const int64_t min_h = gb::kHeights[gb::kNumHeights - 1];
  const int64_t max_tiles = ((R_cap + min_h - 1) / min_h + E) * n_tiles;
  if (max_tiles > INT32_MAX) return NVFP4_ERR_SHAPE;
  // persistent grid: one workgroup per CU on a 256-CU device, a multiple of 8
  int64_t grid = max_tiles < 256 ? max_tiles : 256;
  if (grid >= 8) grid &= ~7ll;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_layout == NVFP4MOE_W_KN)
    gb::bf16_grouped_gemm_kernel<true><<<(unsigned)grid, gb::kThreads, 0, s>>>(
        a, a_map, a_div, (int)a_rows, expert_offsets, E, (int)R_cap, w, (int)N, (int)K, c);
  else
    gb::bf16_grouped_gemm_kernel<false><<<(unsigned)grid, gb::kThreads, 0, s>>>(
        a, a_map, a_div, (int)a_rows, expert_offsets, E, (int)R_cap, w, (int)N, (int)K, c);
  return launch_status();
}

}  // namespace

extern "C" NVFP4MOE_API int bf16_grouped_gemm(const uint16_t* a, const int32_t* expert_offsets,
                                              int32_t E, int64_t R_cap, const uint16_t* w,
                                              int32_t w_layout, int64_t N, int64_t K, float* c,
                                              void* stream) {
  return launch_bf16_grouped_gemm(a, R_cap, nullptr, 1, expert_offsets, E, R_cap, w, w_layout, N, K,
                                  c, stream);
}

extern "C" NVFP4MOE_API int bf16_grouped_gemm_gather(const uint16_t* a, int64_t T,
                                                     const int32_t* row_to_tk, int32_t k,
                                                     const int32_t* expert_offsets, int32_t E,
                                                     int64_t R_cap, const uint16_t* w,
                                                     int32_t w_layout, int64_t N, int64_t K,
                                                     float* c, void* stream) {
  if (k < 1 || k > NVFP4MOE_MAX_TOPK) return NVFP4_ERR_SHAPE;
  if (R_cap > 0 && !row_to_tk) return NVFP4_ERR_NULL;
  return launch_bf16_grouped_gemm(a, T, row_to_tk, k, expert_offsets, E, R_cap, w, w_layout, N, K,
                                  c, stream);
}
