// NVFP4 quantisation kernels for gfx950: per-row quantisation, the MoE
// route + permute + quantise pass, and the weighted SwiGLU + quantise pass.
//
// Method (miniTE pages): per-token scaling (blog "miniTE NVFP4",
// yuxiaoba.github.io, §Follow the numerical execution path); amax taken while
// the permutation or the weighted SwiGLU reads the row, and the scale layout
// written by the quantiser itself, in contiguous expert-grouped buffers with
// device-side offsets (same page, §Two complementary interventions).
//
// Layout of the work: one 64-lane wavefront owns one row.  Lane l holds the 8
// elements [c*512 + 8l, c*512 + 8l + 8) of every 512-element chunk c, loaded
// with one 16-byte load per chunk (a wavefront reads 1 KiB of bf16 contiguous
// per load instruction).  A 16-element block is held by the lane pair (2j,
// 2j+1), so the block amax is one xor-shuffle and the row amax a wavefront
// reduction: the row is read from HBM exactly once.  Codes of 8 elements pack
// into one 32-bit word per lane, so every code store of a wavefront writes 256
// contiguous bytes; four block scales pack into one word.
#include "common.h"

#include <algorithm>
#include <mutex>

namespace nvfp4moe {

constexpr int kRowsPerBlock = 4;           // wavefronts (rows) per 256-thread workgroup
constexpr int kChunk = 512;                // elements per wavefront per 16-byte-per-lane load

// ------------------------------------------------------------------ row quantiser
template <int NCH>
struct RowCodes {
  uint32_t q[NCH];   // packed E2M1 codes of this lane's 8 elements, chunk c
  uint32_t b[NCH];   // E4M3 code of this lane's block, chunk c
  float s;           // row scale (same in every lane)
};

// x[c][j] is element c*512 + 8*lane + j of the row; lanes past the end of the
// row hold zeros.  Follows the definition step by step with IEEE FP32 ops
// (the library is built with -ffp-contract=off, and '/' is correctly rounded).
template <int NCH>
__device__ __forceinline__ void quantize_lane_row(const float (&x)[NCH][8], RowCodes<NCH>& o) {
  float bm[NCH];
  float am = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(x[c][j]));
    bm[c] = fmaxf(m, __shfl_xor(m, 1, kWave));   // block of 16 = lane pair
    am = fmaxf(am, m);
  }
  const float a = wave_max(am);
  const float s = a / 2688.0f;
  const float six_s = 6.0f * s;
  o.s = s;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t b = (s != 0.0f) ? e4m3_encode_nonneg(bm[c] / six_s) : 0u;
    const float d = e4m3_decode_nonneg(b) * s;
    float r[8];
    // fl(x / d) with one division per block: y = fl(1/d), q = fl(x*y),
    // e = x - q*d (exact, one FMA), fl(q + e*y) is the correctly rounded
    // quotient (Markstein) while every value involved is a normal number.  With
    // the block maximum at least 2^-80, d, 1/d and, wherever the quotient is
    // near an E2M1 rounding tie, q and e are normal; far from the ties any
    // small error leaves the code unchanged.  Otherwise (or for an infinity or
    // NaN in the block) divide.  Checked against correctly rounded division on
    // 2e7 quotients placed around every E2M1 tie.
    bool fast = d == 0.0f || bm[c] >= 0x1p-80f;
#pragma unroll
    for (int j = 0; j < 8; ++j) fast = fast && __builtin_isfinite(x[c][j]);
    if (__all(fast)) {
      const float y = 1.0f / (d != 0.0f ? d : 1.0f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float q = x[c][j] * y;
        const float e = __builtin_fmaf(-q, d, x[c][j]);
        const float q2 = __builtin_fmaf(e, y, q);
        // the sign comes from x: the chain turns -0 into +0 (and a zero d
        // gives a zero of x's sign)
        r[j] = __builtin_copysignf(d != 0.0f ? q2 : 0.0f, x[c][j]);
      }
    } else {
      const float dd = d != 0.0f ? d : 1.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = d != 0.0f ? x[c][j] / dd : x[c][j] * 0.0f;
    }
    o.q[c] = e2m1_pack8(r);
    o.b[c] = b;
  }
}

// Block scales leave packed four per 32-bit word.  When K % 64 == 0, lane L
// collects the four scales 4L..4L+3 (chunk L/8, owned by lanes 8(L%8) + 0, 2,
// 4, 6) once per row, so a row's scales are written by lanes 0..K/64-1 with
// one store instruction (up to 256 bytes) instead of 32 bytes per chunk.
template <int NCH>
__device__ __forceinline__ uint32_t gather_scale_word(const RowCodes<NCH>& o, int c0) {
  const int lane = lane_id();
  const int w = c0 * 8 + lane;                 // word index handled by this lane
  const int cw = w >> 3;                       // chunk of that word
  const int src = (w & 7) * 8;                 // first owning lane
  uint32_t word = 0;
#pragma unroll
  for (int cc = 0; cc < 8 && c0 + cc < NCH; ++cc) {
    const uint32_t b0 = __shfl(o.b[c0 + cc], src, kWave);
    const uint32_t b1 = __shfl(o.b[c0 + cc], src + 2, kWave);
    const uint32_t b2 = __shfl(o.b[c0 + cc], src + 4, kWave);
    const uint32_t b3 = __shfl(o.b[c0 + cc], src + 6, kWave);
    if (cw == c0 + cc) word = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }
  return word;
}

// Writes one quantised row.  Codes: one 32-bit word per lane per chunk (a
// wavefront store covers 256 contiguous bytes).  sw[r] are the gathered
// scale words (rounds of 64 words), used when K % 64 == 0; otherwise even
// lanes store one scale byte each.
template <int NCH>
__device__ __forceinline__ void store_row(const RowCodes<NCH>& o, const uint32_t (&sw)[(NCH + 7) / 8],
                                         int K, int64_t row, uint8_t* __restrict__ codes,
                                         uint8_t* __restrict__ bscales,
                                         float* __restrict__ rscales) {
  const int lane = lane_id();
  uint8_t* crow = codes + row * (int64_t)(K / 2);
  uint8_t* brow = bscales + row * (int64_t)(K / 16);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int base = c * kChunk + lane * 8;
    if (base < K) *reinterpret_cast<uint32_t*>(crow + base / 2) = o.q[c];
  }
  if ((K & 63) == 0) {
#pragma unroll
    for (int r = 0; r < (NCH + 7) / 8; ++r) {
      const int w = r * 64 + lane;
      if (w * 64 < K) *reinterpret_cast<uint32_t*>(brow + 4 * w) = sw[r];
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int base = c * kChunk + lane * 8;
      if (base < K && (lane & 1) == 0) brow[base / 16] = (uint8_t)o.b[c];
    }
  }
  if (lane == 0) rscales[row] = o.s;
}

// Writes one quantised row in the K-tiled layout of a group of G rows:
// codes [rows/G][K/64][G][32 B], block scales [rows/G][K/64][G][4 B].  The 64
// elements of K-slab kc of a row are its 32 code bytes and its 4 block scales,
// so the slab of G consecutive rows is one contiguous block (what the grouped
// GEMM reads per K-step).  Requires K % 64 == 0.
template <int NCH>
__device__ __forceinline__ void store_row_tiled(const RowCodes<NCH>& o,
                                               const uint32_t (&sw)[(NCH + 7) / 8], int K,
                                               int64_t row, int64_t G, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ bscales,
                                               float* __restrict__ rscales) {
  const int lane = lane_id();
  const int64_t g = row / G, rr = row - g * G;
  const int64_t slab0 = g * (int64_t)(K >> 6);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int base = c * kChunk + lane * 8;
    if (base < K)
      *reinterpret_cast<uint32_t*>(codes + ((slab0 + (base >> 6)) * G + rr) * 32 + ((base & 63) >> 1)) = o.q[c];
  }
#pragma unroll
  for (int r = 0; r < (NCH + 7) / 8; ++r) {
    const int w = r * 64 + lane;
    if (w * 64 < K) *reinterpret_cast<uint32_t*>(bscales + ((slab0 + w) * G + rr) * 4) = sw[r];
  }
  if (lane == 0) rscales[row] = o.s;
}

template <int NCH>
__device__ __forceinline__ void pack_scales(const RowCodes<NCH>& o, uint32_t (&sw)[(NCH + 7) / 8]) {
#pragma unroll
  for (int r = 0; r < (NCH + 7) / 8; ++r) sw[r] = gather_scale_word<NCH>(o, r * 8);
}

template <int NCH>
__device__ __forceinline__ void load_bf16_raw(const uint16_t* __restrict__ xrow, int K, uint4 (&raw)[NCH]) {
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int base = c * kChunk + lane * 8;
    raw[c] = base < K ? *reinterpret_cast<const uint4*>(xrow + base) : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int NCH>
__device__ __forceinline__ void unpack_bf16(const uint4 (&raw)[NCH], float (&x)[NCH][8]) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint4 v = raw[c];
    x[c][0] = bf16_lo(v.x); x[c][1] = bf16_hi(v.x);
    x[c][2] = bf16_lo(v.y); x[c][3] = bf16_hi(v.y);
    x[c][4] = bf16_lo(v.z); x[c][5] = bf16_hi(v.z);
    x[c][6] = bf16_lo(v.w); x[c][7] = bf16_hi(v.w);
  }
}

template <int NCH>
__device__ __forceinline__ void load_bf16_row(const uint16_t* __restrict__ xrow, int K,
                                              float (&x)[NCH][8]) {
  uint4 raw[NCH];
  load_bf16_raw<NCH>(xrow, K, raw);
  unpack_bf16<NCH>(raw, x);
}

// ------------------------------------------------------------------ contiguous-lane rows
// Rows of K = 1024 * BPL elements (BPL = 1, 2, 4): lane l holds elements
// [16 BPL l, 16 BPL (l + 1)), i.e. BPL whole scale blocks, so a block's maximum
// needs no shuffle and a lane's codes (8 BPL bytes) and block scales (BPL
// bytes) are contiguous: a routed row leaves in one code store and one scale
// store per lane.  Same arithmetic as quantize_lane_row.
template <int BPL>
struct RowCodesC {
  uint32_t q[2 * BPL];   // packed E2M1 codes of the lane's blocks, 8 per word
  uint32_t b[BPL];       // E4M3 code of each block
  float s;               // row scale (same in every lane)
};

template <int BPL>
__device__ __forceinline__ void load_bf16_c(const uint16_t* __restrict__ xrow, uint4 (&raw)[2 * BPL]) {
  const uint4* p = reinterpret_cast<const uint4*>(xrow + 16 * BPL * lane_id());
#pragma unroll
  for (int u = 0; u < 2 * BPL; ++u) raw[u] = p[u];
}

// codes of the 16 elements of one block: fl(x / d) by the quotient rules of
// quantize_lane_row (one division per block where the values allow it)
__device__ __forceinline__ void block_codes16(const float* x, float d, float bmax, uint32_t& w0,
                                              uint32_t& w1) {
  float r[16];
  bool fast = d == 0.0f || bmax >= 0x1p-80f;
#pragma unroll
  for (int j = 0; j < 16; ++j) fast = fast && __builtin_isfinite(x[j]);
  if (__all(fast)) {
    const float y = 1.0f / (d != 0.0f ? d : 1.0f);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float q = x[j] * y;
      const float e = __builtin_fmaf(-q, d, x[j]);
      const float q2 = __builtin_fmaf(e, y, q);
      r[j] = __builtin_copysignf(d != 0.0f ? q2 : 0.0f, x[j]);
    }
  } else {
    const float dd = d != 0.0f ? d : 1.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = d != 0.0f ? x[j] / dd : x[j] * 0.0f;
  }
  w0 = e2m1_pack8(*reinterpret_cast<const float(*)[8]>(r));
  w1 = e2m1_pack8(*reinterpret_cast<const float(*)[8]>(r + 8));
}

template <int BPL>
__device__ __forceinline__ void quantize_lane_row_c(const uint4 (&raw)[2 * BPL], RowCodesC<BPL>& o) {
  float x[BPL][16];
#pragma unroll
  for (int u = 0; u < 2 * BPL; ++u) {
    float* v = &x[u >> 1][8 * (u & 1)];
    v[0] = bf16_lo(raw[u].x); v[1] = bf16_hi(raw[u].x);
    v[2] = bf16_lo(raw[u].y); v[3] = bf16_hi(raw[u].y);
    v[4] = bf16_lo(raw[u].z); v[5] = bf16_hi(raw[u].z);
    v[6] = bf16_lo(raw[u].w); v[7] = bf16_hi(raw[u].w);
  }
  float bm[BPL];
  float am = 0.0f;
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, __builtin_fabsf(x[b][j]));
    bm[b] = m;
    am = fmaxf(am, m);
  }
  const float a = wave_max(am);
  const float s = a / 2688.0f;
  const float six_s = 6.0f * s;
  o.s = s;
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const uint32_t code = (s != 0.0f) ? e4m3_encode_nonneg(bm[b] / six_s) : 0u;
    const float d = e4m3_decode_nonneg(code) * s;
    block_codes16(x[b], d, bm[b], o.q[2 * b], o.q[2 * b + 1]);
    o.b[b] = code;
  }
}

template <int BPL>
__device__ __forceinline__ void store_row_c(const RowCodesC<BPL>& o, int K, int64_t row,
                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ bscales,
                                           float* __restrict__ rscales) {
  const int lane = lane_id();
  uint8_t* crow = codes + row * (int64_t)(K / 2) + 8 * BPL * lane;
  uint8_t* brow = bscales + row * (int64_t)(K / 16) + BPL * lane;
  if constexpr (BPL == 1) {
    *reinterpret_cast<uint2*>(crow) = make_uint2(o.q[0], o.q[1]);
    *brow = (uint8_t)o.b[0];
  } else if constexpr (BPL == 2) {
    *reinterpret_cast<uint4*>(crow) = make_uint4(o.q[0], o.q[1], o.q[2], o.q[3]);
    *reinterpret_cast<uint16_t*>(brow) = (uint16_t)(o.b[0] | (o.b[1] << 8));
  } else {
    static_assert(BPL == 4, "1, 2 or 4 blocks per lane");
    *reinterpret_cast<uint4*>(crow) = make_uint4(o.q[0], o.q[1], o.q[2], o.q[3]);
    *reinterpret_cast<uint4*>(crow + 16) = make_uint4(o.q[4], o.q[5], o.q[6], o.q[7]);
    *reinterpret_cast<uint32_t*>(brow) = o.b[0] | (o.b[1] << 8) | (o.b[2] << 16) | (o.b[3] << 24);
  }
  if (lane == 0) rscales[row] = o.s;
}

// ------------------------------------------------------------------ kernels
template <int NCH>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int K, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ bscales, float* __restrict__ rscales) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  float v[NCH][8];
  load_bf16_row<NCH>(x + row * (int64_t)K, K, v);
  RowCodes<NCH> o;
  quantize_lane_row<NCH>(v, o);
  uint32_t sw[(NCH + 7) / 8];
  pack_scales<NCH>(o, sw);
  store_row<NCH>(o, sw, K, row, codes, bscales, rscales);
}

// rows of 1024 * BPL elements with contiguous lanes
template <int BPL>
__global__ __launch_bounds__(256) void quantize_rows_c_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int K, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ bscales, float* __restrict__ rscales) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint4 raw[2 * BPL];
  load_bf16_c<BPL>(x + row * (int64_t)K, raw);
  RowCodesC<BPL> o;
  quantize_lane_row_c<BPL>(raw, o);
  store_row_c<BPL>(o, K, row, codes, bscales, rscales);
}

template <int NCH>
__global__ __launch_bounds__(256) void quantize_rows_tiled_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int K, int64_t G, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ bscales, float* __restrict__ rscales) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  float v[NCH][8];
  load_bf16_row<NCH>(x + row * (int64_t)K, K, v);
  RowCodes<NCH> o;
  quantize_lane_row<NCH>(v, o);
  uint32_t sw[(NCH + 7) / 8];
  pack_scales<NCH>(o, sw);
  store_row_tiled<NCH>(o, sw, K, row, G, codes, bscales, rscales);
}

// Route + permute + quantise in two launches.
//
// The rank pass: workgroup c (16 wavefronts) takes chunk c of 2^L routing
// entries (L = 11 or 12, chosen per launch by plan_chunk_log).  Each
// wavefront ranks its 2^L / 16 entries in passes of 64 consecutive ones by
// ballot matching on the expert id, keeping a running count per expert in
// LDS; an exclusive scan of those counts over the wavefronts gives every entry
// its stable rank among the chunk's entries of its expert (entry order: token,
// then slot).  The ranks go to the workspace and the chunk's counts per expert
// to the table, cnt[c][e].  Workgroups are independent; the launch boundary
// publishes the results.
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanChunkLogMin = 11;     // 2048 routing entries per chunk: two passes per wavefront
constexpr int kPlanChunkLogMax = 12;     // 4096: four passes
constexpr int kCountTable = 4096;        // ints of (chunk, expert) counts the main pass scans

inline int plan_chunks(int64_t n, int lg) { return n > 0 ? (int)((n + (1ll << lg) - 1) >> lg) : 1; }

// The smallest chunk whose count table still fits the main pass (more
// workgroups share the ranking of a short list), else the largest.  (At 4096
// tokens x 8 of 128 experts, chunks of 2048 entries measured best: 1024 gives
// each main-pass workgroup a 4096-int table to scan, 4096 leaves the rank pass
// on 8 workgroups.)
inline int plan_chunk_log(int64_t n, int E) {
  for (int lg = kPlanChunkLogMin; lg < kPlanChunkLogMax; ++lg)
    if ((int64_t)plan_chunks(n, lg) * E <= kCountTable) return lg;
  return kPlanChunkLogMax;
}

__global__ __launch_bounds__(kPlanThreads) void route_rank_kernel(
    const int32_t* __restrict__ ids, int n, int E, int chunk_log, int32_t* __restrict__ cnt_out,
    int32_t* __restrict__ rank_out, int32_t* __restrict__ dev_err) {
  __shared__ int32_t wcnt[kPlanWaves][NVFP4MOE_MAX_EXPERTS];   // per wavefront, then its exclusive prefix
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int passes = (1 << chunk_log) / kPlanThreads;           // passes of 64 per wavefront (<= 4)
  const int base = (blockIdx.x << chunk_log) + wave * 64 * passes;   // this wavefront's entries
  int ev[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = base + 64 * u + lane;
    ev[u] = (u < passes && i < n) ? ids[i] : -1;
  }
  for (int e = lane; e < E; e += kWave) wcnt[wave][e] = 0;   // each wavefront clears its own row
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int lr[4] = {-1, -1, -1, -1};
  bool bad = false;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u >= passes) break;
    const int i = base + 64 * u + lane;
    const int e = ev[u];
    const bool valid = i < n && e >= 0 && e < E;
    bad |= i < n && !valid;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    lr[u] = -1;
    if (valid) {
      const int r = __popcll(peers & lt_mask);
      const int before = wcnt[wave][e];
      lr[u] = before + r;
      if (r == 0) wcnt[wave][e] = before + __popcll(peers);
    }
  }
  if (bad && dev_err) atomicOr(dev_err, NVFP4_DEVERR_BAD_EXPERT);
  __syncthreads();
  // exclusive scan over the wavefronts, per expert; the chunk's counts
  for (int e = tid; e < E; e += kPlanThreads) {
    int acc = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      const int v = wcnt[w][e];
      wcnt[w][e] = acc;
      acc += v;
    }
    cnt_out[blockIdx.x * E + e] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = base + 64 * u + lane;
    if (u < passes && i < n) rank_out[i] = lr[u] >= 0 ? wcnt[wave][ev[u]] + lr[u] : -1;
  }
}

// The main pass.  Workgroup w (8 wavefronts) owns tokens [8w, 8w + 8), one
// per wavefront.  Every load it needs is issued at the start: the count table
// and the token's k expert ids and ranks first, then the token's activations.
// While the activations are in flight the workgroup forms, from the table,
// the expert offsets and the first row of each expert in the chunk(s) its
// entries fall in; an entry's row is that first row plus its rank.  Then the
// token is quantised and written to its k rows.  Workgroup 0 also writes the
// expert offsets.  Every load is issued unconditionally (indices clamped into
// the arrays) and the workgroup barriers order LDS only, so that waiting for
// the routing loads leaves the activations in flight.
constexpr int kQpWaves = 8;
constexpr int kQpThreads = kQpWaves * 64;
constexpr int kQpExp = NVFP4MOE_MAX_EXPERTS / kQpThreads;   // experts per thread (2)

// workgroup barrier for LDS only: global loads in flight are not waited for
__device__ __forceinline__ void lds_only_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int NCH, int BPL>
__global__ __launch_bounds__(kQpThreads) void quantize_permute_kernel(
    const uint16_t* __restrict__ x, int64_t T, int K, const int32_t* __restrict__ ids, int k, int E,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ rank, int nchunks, int chunk_log,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ bscales, float* __restrict__ rscales,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_tk, int32_t* __restrict__ tk_to_row) {
  __shared__ int32_t sbase[2][NVFP4MOE_MAX_EXPERTS];   // first row of expert e in chunk c0, c0 + 1
  __shared__ int32_t wsum[kQpWaves];
  __shared__ int32_t tab[kCountTable];                  // the count table
  const int lane = lane_id(), wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kQpWaves + wave;
  const int e0 = (int)((int64_t)blockIdx.x * kQpWaves * k);       // first entry of the group
  const int c0 = e0 >> chunk_log;                                  // its chunk
  const int n = (int)(T * k);                                      // routing entries (T >= 1)
  const int ntab = nchunks * E;

  // every load first: the count table and this token's entries, then its activations
  int tv[kCountTable / kQpThreads];             // the table, 8 independent loads per thread
#pragma unroll
  for (int u = 0; u < kCountTable / kQpThreads; ++u) tv[u] = cnt[min(u * kQpThreads + tid, ntab - 1)];
  const int my_i = (int)(t * k) + lane;
  const bool mine = t < T && lane < k;          // lane < k holds entry my_i of this token
  const int my_e = ids[min(my_i, n - 1)];
  const int my_r = rank[min(my_i, n - 1)];
  constexpr bool kC = BPL > 0;                 // contiguous-lane rows
  uint4 raw[kC ? 2 * BPL : NCH];
  const int64_t tl = min(t, T - 1);
  if constexpr (kC) load_bf16_c<BPL>(x + tl * (int64_t)K, raw);
  else load_bf16_raw<NCH>(x + tl * (int64_t)K, K, raw);

  // the table: per expert the total and the entries in chunks before c0, c0 + 1
#pragma unroll
  for (int u = 0; u < kCountTable / kQpThreads; ++u) {
    const int i = u * kQpThreads + tid;
    tab[i] = i < ntab ? tv[u] : 0;
  }
  lds_only_barrier();
  int tot[kQpExp], b0[kQpExp], b1[kQpExp];
#pragma unroll
  for (int u = 0; u < kQpExp; ++u) { tot[u] = 0; b0[u] = 0; b1[u] = 0; }
  for (int c = 0; c < nchunks; ++c) {
#pragma unroll
    for (int u = 0; u < kQpExp; ++u) {
      const int e = kQpExp * tid + u;
      const int v = e < E ? tab[c * E + e] : 0;
      tot[u] += v;
      if (c < c0) b0[u] += v;
      if (c <= c0) b1[u] += v;
    }
  }
  // expert offsets: exclusive scan of the totals over experts
  int mine_tot = 0;
#pragma unroll
  for (int u = 0; u < kQpExp; ++u) mine_tot += tot[u];
  int incl = mine_tot;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  lds_only_barrier();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int off_e = before + incl - mine_tot;   // offset of expert kQpExp * tid
#pragma unroll
  for (int u = 0; u < kQpExp; ++u) {
    const int e = kQpExp * tid + u;
    if (e < E) {
      sbase[0][e] = off_e + b0[u];
      sbase[1][e] = off_e + b1[u];
      if (blockIdx.x == 0) offsets[e] = off_e;
    }
    off_e += tot[u];
  }
  if (blockIdx.x == 0 && tid == kQpThreads - 1) offsets[E] = before + incl;
  lds_only_barrier();
  if (t >= T) return;
  // the rows of this token's entries (a rank >= 0 marks a valid expert id)
  int row = -1;
  if (mine) {
    if (my_r >= 0) row = sbase[(my_i >> chunk_log) - c0][my_e] + my_r;
    tk_to_row[my_i] = row;
    if (row >= 0) row_to_tk[row] = my_i;
  }
  // the token's codes (its activations have landed meanwhile)
  RowCodes<NCH> o;
  RowCodesC<kC ? BPL : 1> oc;
  uint32_t sw[(NCH + 7) / 8];
  if constexpr (kC) {
    quantize_lane_row_c<BPL>(raw, oc);
  } else {
    float v[NCH][8];
    unpack_bf16<NCH>(raw, v);
    quantize_lane_row<NCH>(v, o);
    pack_scales<NCH>(o, sw);
  }
  for (int slot = 0; slot < k; ++slot) {
    const int r = __shfl(row, slot, kWave);
    if (r >= 0) {
      if constexpr (kC) store_row_c<BPL>(oc, K, r, codes, bscales, rscales);
      else store_row<NCH>(o, sw, K, r, codes, bscales, rscales);
    }
  }
}

// Long routing lists (a count table too large for every workgroup of the
// main pass to scan), long rows, or no tokens: the ranks as above, then one
// workgroup turns the table into first rows,
//   base[c][e] = offsets[e] + (entries of e in chunks before c),
// in place and writes the offsets; the main pass then needs no scan at all.

__global__ __launch_bounds__(kPlanThreads) void route_scan_kernel(
    int32_t* __restrict__ table, int nchunks, int E, int32_t* __restrict__ offsets) {
  __shared__ int32_t part[kPlanThreads];
  __shared__ int32_t wsum[kPlanWaves];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  // thread (e, p), P = 1024 / E threads per expert, sums chunks [p cpt, (p + 1) cpt)
  const int P = kPlanThreads / E, cpt = (nchunks + P - 1) / P;
  const int e = tid / P, p = tid - e * P;
  const int c_lo = min(nchunks, p * cpt), c_hi = min(nchunks, (p + 1) * cpt);
  int sum = 0;
  if (e < E)
    for (int c = c_lo; c < c_hi; ++c) sum += table[(int64_t)c * E + e];
  part[tid] = sum;
  __syncthreads();
  int pre_p = 0, tot = 0;
  if (e < E) {
    for (int q = 0; q < P; ++q) {
      const int v = part[e * P + q];
      if (q < p) pre_p += v;
      tot += v;
    }
  }
  // offsets: exclusive scan over experts of the totals, carried by thread (e, 0)
  const int mine = (e < E && p == 0) ? tot : 0;
  int incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();   // also: every read of part[] above is done
  int wbefore = 0;
  for (int w = 0; w < wave; ++w) wbefore += wsum[w];
  if (e < E && p == 0) part[e] = wbefore + incl - mine;
  __syncthreads();
  if (e < E) {
    const int off_e = part[e];
    if (p == 0) offsets[e] = off_e;
    int acc = off_e + pre_p;
    for (int c = c_lo; c < c_hi; ++c) {
      const int64_t at = (int64_t)c * E + e;
      const int v = table[at];
      table[at] = acc;
      acc += v;
    }
  }
  if (tid == kPlanThreads - 1) offsets[E] = wbefore + incl;
}

// Main pass over first rows: one wavefront per token, independent of every
// other.  Lanes s < k read entry t k + s (expert id and rank) and the first
// row of its expert in its chunk; the token is quantised once and written to
// its k rows.
constexpr int kQrWaves = 4;

template <int NCH, int BPL>
__global__ __launch_bounds__(kQrWaves * 64) void quantize_permute_rows_kernel(
    const uint16_t* __restrict__ x, int64_t T, int K, const int32_t* __restrict__ ids, int k, int E,
    const int32_t* __restrict__ base, const int32_t* __restrict__ rank, int chunk_log,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ bscales, float* __restrict__ rscales,
    int32_t* __restrict__ row_to_tk, int32_t* __restrict__ tk_to_row) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * kQrWaves + wave;
  if (t >= T) return;
  constexpr bool kC = BPL > 0;                 // contiguous-lane rows
  uint4 raw[kC ? 2 * BPL : NCH];
  if constexpr (kC) load_bf16_c<BPL>(x + t * (int64_t)K, raw);
  else load_bf16_raw<NCH>(x + t * (int64_t)K, K, raw);
  int row = -1;
  if (lane < k) {
    const int i = (int)(t * k) + lane;
    const int e = ids[i], r = rank[i];
    if (r >= 0) row = base[(int64_t)(i >> chunk_log) * E + e] + r;
    tk_to_row[i] = row;
    if (row >= 0) row_to_tk[row] = i;
  }
  RowCodes<NCH> o;
  RowCodesC<kC ? BPL : 1> oc;
  uint32_t sw[(NCH + 7) / 8];
  if constexpr (kC) {
    quantize_lane_row_c<BPL>(raw, oc);
  } else {
    float v[NCH][8];
    unpack_bf16<NCH>(raw, v);
    quantize_lane_row<NCH>(v, o);
    pack_scales<NCH>(o, sw);
  }
  for (int slot = 0; slot < k; ++slot) {
    const int r = __shfl(row, slot, kWave);
    if (r >= 0) {
      if constexpr (kC) store_row_c<BPL>(oc, K, r, codes, bscales, rscales);
      else store_row<NCH>(o, sw, K, r, codes, bscales, rscales);
    }
  }
}

// Weighted SwiGLU on one routed row, evaluated in FP64 and rounded once to
// FP32, then the row quantiser; the amax is taken on the values just made.
template <int NCH>
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(
    const float* __restrict__ gu, int64_t R_cap, int I, const int32_t* __restrict__ offsets, int E,
    const float* __restrict__ topk_w, const int32_t* __restrict__ row_to_tk,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ bscales, float* __restrict__ rscales,
    float* __restrict__ h_out) {
  __shared__ double exp2_tab[64];
  stage_exp2_table(exp2_tab);
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= offsets[E] || r >= R_cap) return;
  const int lane = lane_id();
  const float* grow = gu + r * (int64_t)(2 * I);
  float w = 1.0f;
  if (topk_w) {   // the router weight of the row's (token, slot); a bad map entry gives 0
    const int32_t i = row_to_tk[r];
    w = (i >= 0 && i < R_cap) ? topk_w[i] : 0.0f;
  }
  // SwiGLU of one element: float64 (silu(g) as g times the sigmoid), then
  // times u and the router weight, rounded once to float
  auto swiglu = [&](float gf, float uf) __attribute__((always_inline)) -> float {
    double hv = ((double)gf * sigmoid_f64(gf, exp2_tab)) * (double)uf;
    if (topk_w) hv = hv * (double)w;
    return (float)hv;
  };
  // The quantiser's layout gives lane l elements c*512 + 8l .. +7; a last chunk
  // of at most 256 elements would leave half the lanes idle in the float64
  // work, so there lane l computes elements 4l .. 4l+3 and the values move to
  // their lanes by shuffles (same arithmetic, same results).
  const int tail = I - (NCH - 1) * kChunk;             // elements in the last chunk
  const bool split_tail = tail <= kChunk / 2;
  float h[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c == NCH - 1 && split_tail) {
      const int b4 = c * kChunk + lane * 4;
      float hb[4] = {0.f, 0.f, 0.f, 0.f};
      if (lane * 4 < tail) {
        const float4 g4 = *reinterpret_cast<const float4*>(grow + b4);
        const float4 u4 = *reinterpret_cast<const float4*>(grow + I + b4);
        hb[0] = swiglu(g4.x, u4.x);
        hb[1] = swiglu(g4.y, u4.y);
        hb[2] = swiglu(g4.z, u4.z);
        hb[3] = swiglu(g4.w, u4.w);
        if (h_out)
          *reinterpret_cast<float4*>(h_out + r * (int64_t)I + b4) = make_float4(hb[0], hb[1], hb[2], hb[3]);
      }
      const bool mine = lane * 8 < tail;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __shfl(hb[j], 2 * lane, kWave);       // from lane 2l: elements 8l .. 8l+3
        const float hi = __shfl(hb[j], 2 * lane + 1, kWave);   // from lane 2l+1: 8l+4 .. 8l+7
        h[c][j] = mine ? lo : 0.0f;
        h[c][4 + j] = mine ? hi : 0.0f;
      }
      continue;
    }
    const int base = c * kChunk + lane * 8;
    if (base < I) {
      const float4 g0 = *reinterpret_cast<const float4*>(grow + base);
      const float4 g1 = *reinterpret_cast<const float4*>(grow + base + 4);
      const float4 u0 = *reinterpret_cast<const float4*>(grow + I + base);
      const float4 u1 = *reinterpret_cast<const float4*>(grow + I + base + 4);
      const float gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float us[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) h[c][j] = swiglu(gs[j], us[j]);
      if (h_out) {
        float* hrow = h_out + r * (int64_t)I + base;
        *reinterpret_cast<float4*>(hrow) = make_float4(h[c][0], h[c][1], h[c][2], h[c][3]);
        *reinterpret_cast<float4*>(hrow + 4) = make_float4(h[c][4], h[c][5], h[c][6], h[c][7]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[c][j] = 0.0f;
    }
  }
  RowCodes<NCH> o;
  quantize_lane_row<NCH>(h, o);
  uint32_t sw[(NCH + 7) / 8];
  pack_scales<NCH>(o, sw);
  store_row<NCH>(o, sw, I, r, codes, bscales, rscales);
}

// FP32 rows (the weighted SwiGLU output of the fused gate_up GEMM): the row
// quantiser on rows [0, min(offsets[E], rows)) (all rows when offsets is null);
// the row amax is taken in registers while the row is read for quantisation.
template <int NCH>
__global__ __launch_bounds__(256) void quantize_rows_f32_kernel(
    const float* __restrict__ x, int64_t rows, int K, const int32_t* __restrict__ offsets, int E,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ bscales, float* __restrict__ rscales) {
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= rows || (offsets && r >= offsets[E])) return;
  const int lane = lane_id();
  const float* xrow = x + r * (int64_t)K;
  float v[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int base = c * kChunk + lane * 8;
    if (base < K) {
      const float4 a = *reinterpret_cast<const float4*>(xrow + base);
      const float4 b = *reinterpret_cast<const float4*>(xrow + base + 4);
      v[c][0] = a.x; v[c][1] = a.y; v[c][2] = a.z; v[c][3] = a.w;
      v[c][4] = b.x; v[c][5] = b.y; v[c][6] = b.z; v[c][7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[c][j] = 0.0f;
    }
  }
  RowCodes<NCH> o;
  quantize_lane_row<NCH>(v, o);
  uint32_t sw[(NCH + 7) / 8];
  pack_scales<NCH>(o, sw);
  store_row<NCH>(o, sw, K, r, codes, bscales, rscales);
}

// ------------------------------------------------------------------ quantisation along tokens
// The token blocks of the weight gradient: kofs[e] = the first 64-token step of
// expert e's slab, each expert taking max(1, ceil(rows / 64)) steps.  One
// workgroup (E <= 1024).
__global__ __launch_bounds__(1024) void token_blocks_kernel(const int32_t* __restrict__ offsets, int E,
                                                            int32_t* __restrict__ kofs) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int v = tid < E ? max(1, (offsets[tid + 1] - offsets[tid] + 63) >> 6) : 0;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  if (tid < E) kofs[tid] = before + incl - v;
  if (tid == E - 1) kofs[E] = before + incl;
}

// Workgroup (column chunk, expert e): 256 columns c0 .. c0 + 255 of the
// expert's rows, thread (cg = tid % 32, rg = tid / 32) on the 8 columns
// c0 + 8 cg .. +7.  Pass 1: column maxima over the expert's rows (row groups
// rg, rg + 8, ...), combined in LDS; s = amax / 2688 per column.  Pass 2: per
// block of 16 tokens (blocks rg, rg + 8, ...) the 16 x 8 values, each
// column's block scale and codes by the row quantiser's arithmetic, written
// as 8 code bytes and one scale byte per column; blocks past the expert's
// rows are zero padding (scale 0, codes 0).
template <bool F32IN, bool KTILED>
__global__ __launch_bounds__(256) void quantize_tokens_kernel(
    const void* __restrict__ x, int64_t x_rows, int C, const int32_t* __restrict__ row_to_tk, int k,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ kofs, int64_t Kp,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ bscales, float* __restrict__ rscales) {
  __shared__ float cmax[8][256];
  const int tid = threadIdx.x, cg = tid & 31, rg = tid >> 5;
  const int e = blockIdx.y;
  const int c = (int)blockIdx.x * 256 + 8 * cg;                  // first of the thread's 8 columns
  const int r0 = offsets[e], n = offsets[e + 1] - r0;
  const int kb0 = kofs[e], nblk = (kofs[e + 1] - kb0) * 4;      // blocks of 16 tokens in the slab
  if (kb0 < 0 || kofs[e + 1] < kb0 || (int64_t)(kofs[e + 1]) * 64 > Kp) return;   // slab outside the buffer: skipped
  auto load8 = [&](int r, float (&v)[8]) __attribute__((always_inline)) {
    int64_t xr = r0 + r;
    // token-order input: the routing map has x_rows * k entries; a bad offset or
    // map entry reads a wrong row, never one outside x
    if (row_to_tk) xr = row_to_tk[min(max(xr, (int64_t)0), x_rows * k - 1)] / k;
    xr = xr < 0 ? 0 : (xr >= x_rows ? x_rows - 1 : xr);
    if constexpr (F32IN) {
      const float* p = static_cast<const float*>(x) + xr * C + c;
      const float4 a = *reinterpret_cast<const float4*>(p);
      const float4 b = *reinterpret_cast<const float4*>(p + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + xr * C + c);
      v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
      v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
  };
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = rg; r < n; r += 8) {
    float v[8];
    load8(r, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], __builtin_fabsf(v[j]));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) cmax[rg][8 * cg + j] = m[j];
  __syncthreads();
  float s[8], six_s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float a = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) a = fmaxf(a, cmax[g][8 * cg + j]);
    s[j] = a / 2688.0f;
    six_s[j] = 6.0f * s[j];
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) rscales[(int64_t)e * C + c + j] = s[j];
  }
  for (int b = rg; b < nblk; b += 8) {
    float v[16][8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (16 * b + i < n) load8(16 * b + i, v[i]);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
      }
    }
    const int64_t kpos = (int64_t)kb0 * 64 + 16 * b;             // first token position of the block
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float col[16];
      float bm = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        col[i] = v[i][j];
        bm = fmaxf(bm, __builtin_fabsf(col[i]));
      }
      const uint32_t bs = s[j] != 0.0f ? e4m3_encode_nonneg(bm / six_s[j]) : 0u;
      const float d = e4m3_decode_nonneg(bs) * s[j];
      uint32_t w0, w1;
      block_codes16(col, d, bm, w0, w1);
      const int64_t row = c + j;
      if constexpr (KTILED) {
        const int64_t slab = kpos >> 6;
        const int q = (int)(kpos & 63) >> 4;                     // block within the slab
        *reinterpret_cast<uint2*>(codes + (slab * C + row) * 32 + 8 * q) = make_uint2(w0, w1);
        bscales[(slab * C + row) * 4 + q] = (uint8_t)bs;
      } else {
        *reinterpret_cast<uint2*>(codes + row * (Kp / 2) + kpos / 2) = make_uint2(w0, w1);
        bscales[row * (Kp / 16) + kpos / 16] = (uint8_t)bs;
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch
inline int nch_for(int64_t K) {
  return K <= 512 ? 1 : K <= 1024 ? 2 : K <= 2048 ? 4 : K <= 4096 ? 8 : 16;
}

#define NVFP4_DISPATCH_NCH(K, KERNEL, GRID, STREAM, ...)                                \
  switch (nch_for(K)) {                                                                 \
    case 1: KERNEL<1><<<GRID, 256, 0, STREAM>>>(__VA_ARGS__); break;                    \
    case 2: KERNEL<2><<<GRID, 256, 0, STREAM>>>(__VA_ARGS__); break;                    \
    case 4: KERNEL<4><<<GRID, 256, 0, STREAM>>>(__VA_ARGS__); break;                    \
    case 8: KERNEL<8><<<GRID, 256, 0, STREAM>>>(__VA_ARGS__); break;                    \
    default: KERNEL<16><<<GRID, 256, 0, STREAM>>>(__VA_ARGS__); break;                  \
  }

}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" {

NVFP4MOE_API const char* nvfp4moe_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "a size argument is out of range";
    case NVFP4_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case NVFP4_ERR_WORKSPACE: return "workspace too small";
    case NVFP4_ERR_LAUNCH: return "the HIP runtime reported an error when enqueuing";
    case NVFP4_ERR_ARG: return "an enumerated argument has an unknown value";
    case NVFP4_ERR_SCRATCH:
      return "more routing entries (T * k) than the allocation-free entry point's fixed device scratch holds";
    default: return "unknown status";
  }
}

NVFP4MOE_API int nvfp4moe_abi_version(void) { return NVFP4MOE_ABI_VERSION; }

NVFP4MOE_API int64_t nvfp4moe_bscale_index(int64_t r, int64_t kb, int64_t K, int64_t group_rows) {
  if (r < 0 || K <= 0 || kb < 0 || kb >= K / 16 || group_rows < 0) return -1;
  if (group_rows == 0) return K % 16 ? -1 : r * (K / 16) + kb;
  if (K % 64) return -1;
  const int64_t g = r / group_rows, rr = r - g * group_rows;
  return ((g * (K / 64) + kb / 4) * group_rows + rr) * 4 + kb % 4;
}

NVFP4MOE_API int64_t nvfp4moe_code_index(int64_t r, int64_t i, int64_t K, int64_t group_rows) {
  if (r < 0 || K <= 0 || i < 0 || i >= K || group_rows < 0) return -1;
  if (group_rows == 0) return K % 16 ? -1 : r * (K / 2) + i / 2;
  if (K % 64) return -1;
  const int64_t g = r / group_rows, rr = r - g * group_rows;
  return ((g * (K / 64) + i / 64) * group_rows + rr) * 32 + (i % 64) / 2;
}

NVFP4MOE_API size_t nvfp4moe_permute_workspace_size(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k <= 0 || E <= 0) return 0;
  // the (chunk, expert) count table and a rank per routing entry
  const int64_t n = T * (int64_t)k;
  const size_t bytes = ((size_t)plan_chunks(n, plan_chunk_log(n, E)) * (size_t)E + (size_t)n) * sizeof(int32_t);
  return (bytes + 255) & ~(size_t)255;
}

NVFP4MOE_API size_t nvfp4moe_workspace_size(int32_t op, int64_t T, int32_t E, int32_t k,
                                            int64_t R_max, int64_t N) {
  (void)N;
  switch (op) {
    case NVFP4MOE_OP_QUANTIZE_PERMUTE: return nvfp4moe_permute_workspace_size(T, k, E);
    case NVFP4MOE_OP_QUANTIZE_ROWS:
    case NVFP4MOE_OP_GROUPED_GEMM:
    case NVFP4MOE_OP_SWIGLU_QUANTIZE:
    case NVFP4MOE_OP_UNPERMUTE_COMBINE:
    case NVFP4MOE_OP_BF16_GROUPED_GEMM:
    case NVFP4MOE_OP_SWIGLU_BACKWARD: return 0;
    case NVFP4MOE_OP_GROUPED_GEMM_SWIGLU:
      return R_max < 0 ? 0 : (((size_t)R_max * sizeof(float) + 255) & ~(size_t)255);
    default: return (size_t)-1;
  }
}

NVFP4MOE_API int nvfp4_quantize_rows(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                                     uint8_t* bscales, float* rscales, void* stream) {
  if (rows < 0 || K <= 0 || K % 16 != 0 || K > NVFP4MOE_MAX_K) return NVFP4_ERR_SHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!x || !codes || !bscales || !rscales) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(bscales) || !aligned16(rscales))
    return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  if (K == 1024)
    quantize_rows_c_kernel<1><<<grid, 256, 0, s>>>(x, rows, (int)K, codes, bscales, rscales);
  else if (K == 2048)
    quantize_rows_c_kernel<2><<<grid, 256, 0, s>>>(x, rows, (int)K, codes, bscales, rscales);
  else if (K == 4096)
    quantize_rows_c_kernel<4><<<grid, 256, 0, s>>>(x, rows, (int)K, codes, bscales, rscales);
  else
    NVFP4_DISPATCH_NCH(K, quantize_rows_kernel, grid, s, x, rows, (int)K, codes, bscales, rscales);
  return launch_status();
}

NVFP4MOE_API int nvfp4_quantize_rows_f32(const float* x, int64_t rows, int64_t K,
                                         const int32_t* expert_offsets, int32_t E, uint8_t* codes,
                                         uint8_t* bscales, float* rscales, void* stream) {
  if (rows < 0 || K <= 0 || K % 16 != 0 || K > NVFP4MOE_MAX_K) return NVFP4_ERR_SHAPE;
  if (expert_offsets && (E < 1 || E > NVFP4MOE_MAX_EXPERTS)) return NVFP4_ERR_SHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!x || !codes || !bscales || !rscales) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(bscales) || !aligned16(rscales))
    return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  NVFP4_DISPATCH_NCH(K, quantize_rows_f32_kernel, grid, s, x, rows, (int)K, expert_offsets, E, codes,
                     bscales, rscales);
  return launch_status();
}

NVFP4MOE_API int nvfp4moe_token_blocks(const int32_t* expert_offsets, int32_t E, int32_t* kofs,
                                       void* stream) {
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS) return NVFP4_ERR_SHAPE;
  if (!expert_offsets || !kofs) return NVFP4_ERR_NULL;
  token_blocks_kernel<<<1, 1024, 0, static_cast<hipStream_t>(stream)>>>(expert_offsets, E, kofs);
  return launch_status();
}

NVFP4MOE_API int nvfp4_quantize_tokens(const void* x, int32_t x_dtype, int64_t x_rows, int64_t C,
                                       const int32_t* row_to_tk, int32_t k,
                                       const int32_t* expert_offsets, const int32_t* kofs, int32_t E,
                                       int64_t Kp, int32_t layout, uint8_t* codes, uint8_t* bscales,
                                       float* rscales, void* stream) {
  if (x_dtype != NVFP4_IN_BF16 && x_dtype != NVFP4_IN_F32) return NVFP4_ERR_ARG;
  if (layout != NVFP4_W_ROWMAJOR && layout != NVFP4_W_KTILED) return NVFP4_ERR_ARG;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS || x_rows < 1 || C < 256 || C % 256 != 0 || C > (1 << 20))
    return NVFP4_ERR_SHAPE;
  if (Kp <= 0 || Kp % 64 != 0 || (row_to_tk && (k < 1 || k > NVFP4MOE_MAX_TOPK))) return NVFP4_ERR_SHAPE;
  if (!x || !expert_offsets || !kofs || !codes || !bscales || !rscales) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(bscales) || !aligned16(rscales))
    return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(C / 256), (unsigned)E);
#define QT_LAUNCH(F, KTL)                                                                         \
  quantize_tokens_kernel<F, KTL><<<grid, 256, 0, s>>>(x, x_rows, (int)C, row_to_tk, k, expert_offsets, \
                                                     kofs, Kp, codes, bscales, rscales)
  const bool f32 = x_dtype == NVFP4_IN_F32, kt = layout == NVFP4_W_KTILED;
  if (f32 && kt) QT_LAUNCH(true, true);
  else if (f32) QT_LAUNCH(true, false);
  else if (kt) QT_LAUNCH(false, true);
  else QT_LAUNCH(false, false);
#undef QT_LAUNCH
  return launch_status();
}

NVFP4MOE_API int nvfp4_quantize_rows_tiled(const uint16_t* x, int64_t rows, int64_t K,
                                           int64_t group_rows, uint8_t* codes, uint8_t* bscales,
                                           float* rscales, void* stream) {
  if (rows < 0 || K <= 0 || K % 64 != 0 || K > NVFP4MOE_MAX_K) return NVFP4_ERR_SHAPE;
  if (group_rows <= 0 || rows % group_rows != 0) return NVFP4_ERR_SHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!x || !codes || !bscales || !rscales) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(bscales) || !aligned16(rscales))
    return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  NVFP4_DISPATCH_NCH(K, quantize_rows_tiled_kernel, grid, s, x, rows, (int)K, group_rows, codes,
                     bscales, rscales);
  return launch_status();
}

}  // extern "C"

namespace nvfp4moe {

// The route + permute + quantise pass on a caller-given workspace (the count
// table, then one rank per routing entry; every word is written before it is
// read, so the workspace needs no clearing).
static int quantize_permute_impl(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                 int32_t k, int32_t E, uint8_t* codes, uint8_t* bscales,
                                 float* rscales, int32_t* expert_offsets, int32_t* row_to_tk,
                                 int32_t* tk_to_row, void* workspace, size_t workspace_bytes,
                                 int32_t* dev_err, void* stream) {
  if (T < 0 || H <= 0 || H % 16 != 0 || H > NVFP4MOE_MAX_K) return NVFP4_ERR_SHAPE;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS || k < 1 || k > E || k > NVFP4MOE_MAX_TOPK)
    return NVFP4_ERR_SHAPE;
  // entry indices, plus a chunk's worth past the last, stay in int
  if (T * (int64_t)k > INT32_MAX / 2) return NVFP4_ERR_SHAPE;
  if (!expert_offsets || !workspace) return NVFP4_ERR_NULL;
  if (T > 0 && (!x || !topk_ids || !codes || !bscales || !rscales || !row_to_tk || !tk_to_row))
    return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(bscales) || !aligned16(rscales) ||
      !aligned16(workspace))
    return NVFP4_ERR_ALIGN;
  if (workspace_bytes < nvfp4moe_permute_workspace_size(T, k, E)) return NVFP4_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n = T * (int64_t)k;
  const int chunk_log = plan_chunk_log(n, E);
  const int pchunks = plan_chunks(n, chunk_log);
  int32_t* table = static_cast<int32_t*>(workspace);        // [pchunks][E]
  int32_t* rank = table + (int64_t)pchunks * E;              // [n]
  // rank every entry within its chunk and expert, and count per (chunk, expert)
  route_rank_kernel<<<pchunks, kPlanThreads, 0, s>>>(topk_ids, (int)n, E, chunk_log, table, rank,
                                                     dev_err);
  if (T > 0 && (int64_t)pchunks * E <= kCountTable && H <= 4096) {
    // offsets + first rows from the table in every workgroup, then rows +
    // quantise + scatter
    const unsigned grid = (unsigned)((T + kQpWaves - 1) / kQpWaves);
#define QP_LAUNCH(C, B)                                                                          \
    quantize_permute_kernel<C, B><<<grid, kQpThreads, 0, s>>>(x, T, (int)H, topk_ids, (int)k,     \
        (int)E, table, rank, pchunks, chunk_log, codes, bscales, rscales, expert_offsets,         \
        row_to_tk, tk_to_row)
    // rows of 1024, 2048 or 4096 elements: contiguous lanes; other lengths: strided lanes
    if (H == 1024) QP_LAUNCH(2, 1);
    else if (H == 2048) QP_LAUNCH(4, 2);
    else if (H == 4096) QP_LAUNCH(8, 4);
    else {
      switch (nch_for(H)) {
        case 1: QP_LAUNCH(1, 0); break;
        case 2: QP_LAUNCH(2, 0); break;
        case 4: QP_LAUNCH(4, 0); break;
        default: QP_LAUNCH(8, 0); break;
      }
    }
#undef QP_LAUNCH
    return launch_status();
  }
  // long routing lists, long rows, or no tokens: one workgroup turns the table
  // into first rows and writes the offsets; then rows + quantise + scatter
  // with independent wavefronts
  route_scan_kernel<<<1, kPlanThreads, 0, s>>>(table, pchunks, E, expert_offsets);
  if (T > 0) {
    const unsigned grid = (unsigned)((T + kQrWaves - 1) / kQrWaves);
#define QR_LAUNCH(C, B)                                                                          \
    quantize_permute_rows_kernel<C, B><<<grid, kQrWaves * 64, 0, s>>>(x, T, (int)H, topk_ids,     \
        (int)k, (int)E, table, rank, chunk_log, codes, bscales, rscales, row_to_tk, tk_to_row)
    if (H == 1024) QR_LAUNCH(2, 1);
    else if (H == 2048) QR_LAUNCH(4, 2);
    else if (H == 4096) QR_LAUNCH(8, 4);
    else {
      switch (nch_for(H)) {
        case 1: QR_LAUNCH(1, 0); break;
        case 2: QR_LAUNCH(2, 0); break;
        case 4: QR_LAUNCH(4, 0); break;
        case 8: QR_LAUNCH(8, 0); break;
        default: QR_LAUNCH(16, 0); break;
      }
    }
#undef QR_LAUNCH
  }
  return launch_status();
}

// Scratch of the allocation-free entry point: the workspace of
// quantize_permute_impl for up to NVFP4MOE_NOALLOC_MAX_ENTRIES routing entries
// and NVFP4MOE_MAX_EXPERTS experts, as a device array of the library (each
// device holds its own copy while the process lives).  Host code never passes
// the array's name to a kernel: it stands for the host-side shadow, so the
// device address is looked up once per device and kept in scratch_ptr.
// (A chunk shorter than the largest is only chosen when its table fits
// kCountTable words, which the largest chunk's table bound covers.)
constexpr int64_t kNoAllocWords =
    (int64_t)((NVFP4MOE_NOALLOC_MAX_ENTRIES + (1 << kPlanChunkLogMax) - 1) >> kPlanChunkLogMax) *
        NVFP4MOE_MAX_EXPERTS +
    NVFP4MOE_NOALLOC_MAX_ENTRIES;
static_assert((1 << kPlanChunkLogMax) / kPlanThreads <= 4, "at most four passes of 64 per wavefront");
static_assert((int64_t)((NVFP4MOE_NOALLOC_MAX_ENTRIES + (1 << kPlanChunkLogMax) - 1) >> kPlanChunkLogMax) *
                  NVFP4MOE_MAX_EXPERTS >= kCountTable, "scratch holds a count table of kCountTable words");
static __device__ __align__(256) int32_t scratch[kNoAllocWords];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void* scratch_ptr[kMaxDevices];

// device address of `scratch` on the current device (looked up on the first
// call there); null if the runtime reports an error
static void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace nvfp4moe

extern "C" {

NVFP4MOE_API int nvfp4_quantize_permute(const uint16_t* x, int64_t T, int64_t H,
                                        const int32_t* topk_ids, int32_t k, int32_t E,
                                        uint8_t* codes, uint8_t* bscales, float* rscales,
                                        int32_t* expert_offsets, int32_t* row_to_tk,
                                        int32_t* tk_to_row, void* workspace,
                                        size_t workspace_bytes, int32_t* dev_err, void* stream) {
  return quantize_permute_impl(x, T, H, topk_ids, k, E, codes, bscales, rscales, expert_offsets,
                               row_to_tk, tk_to_row, workspace, workspace_bytes, dev_err, stream);
}

NVFP4MOE_API int nvfp4_quantize_permute_noalloc(const uint16_t* x, int64_t T, int64_t H,
                                                const int32_t* topk_ids, int32_t k, int32_t E,
                                                uint8_t* codes, uint8_t* bscales, float* rscales,
                                                int32_t* expert_offsets, int32_t* row_to_tk,
                                                int32_t* tk_to_row, int32_t* dev_err,
                                                void* stream) {
  if (T < 0 || k < 1) return NVFP4_ERR_SHAPE;
  if (T * (int64_t)k > NVFP4MOE_NOALLOC_MAX_ENTRIES) return NVFP4_ERR_SCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return NVFP4_ERR_LAUNCH;
  return quantize_permute_impl(x, T, H, topk_ids, k, E, codes, bscales, rscales, expert_offsets,
                               row_to_tk, tk_to_row, ws, (size_t)kNoAllocWords * sizeof(int32_t),
                               dev_err, stream);
}

NVFP4MOE_API int swiglu_quantize(const float* gu, int64_t R_cap, int64_t I,
                                 const int32_t* expert_offsets, int32_t E, const float* topk_w,
                                 const int32_t* row_to_tk, uint8_t* codes, uint8_t* bscales,
                                 float* rscales, float* h_out, void* stream) {
  if (R_cap < 0 || I < 16 || I % 16 != 0 || I > NVFP4MOE_MAX_K) return NVFP4_ERR_SHAPE;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS) return NVFP4_ERR_SHAPE;
  if (R_cap == 0) return NVFP4_OK;
  if (!gu || !expert_offsets || !codes || !bscales || !rscales) return NVFP4_ERR_NULL;
  if (topk_w && !row_to_tk) return NVFP4_ERR_NULL;
  if (!aligned16(gu) || !aligned16(codes) || !aligned16(bscales) || !aligned16(rscales) ||
      !aligned16(h_out))
    return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((R_cap + kRowsPerBlock - 1) / kRowsPerBlock));
  NVFP4_DISPATCH_NCH(I, swiglu_quantize_kernel, grid, s, gu, R_cap, (int)I, expert_offsets, E, topk_w,
                     row_to_tk, codes, bscales, rscales, h_out);
  return launch_status();
}

}  // extern "C"
