// Un-permutation with the top-k combine, the gather of token rows to routed
// rows, and the SwiGLU backward, for gfx950.  All three are HBM-bound
// streaming kernels: one 64-lane wavefront per token or routed row, 16-byte
// loads and stores per lane, rows located through the identity maps the
// permutation produced (blog "miniTE NVFP4", yuxiaoba.github.io, §Follow the
// numerical execution path: token and expert identities kept for alignment;
// §Two complementary interventions: device-side metadata, independent
// forward/backward precision).
#include "common.h"

namespace nvfp4moe {

constexpr int kRows = 4;   // wavefronts per 256-thread workgroup

// y[t] = bf16( ((w0 d[r0] + w1 d[r1]) + ...) + w_{k-1} d[r_{k-1}] ), FP32, slot order.
__global__ __launch_bounds__(256) void unpermute_combine_kernel(
    const float* __restrict__ d, int64_t T, int k, int H, const int32_t* __restrict__ tk_to_row,
    const float* __restrict__ topk_w, uint16_t* __restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * kRows + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const int my_row = lane < k ? tk_to_row[t * k + lane] : -1;
  const float my_w = (lane < k && topk_w) ? topk_w[t * k + lane] : 1.0f;
  // The loops are wave-uniform (every lane runs every slot) because the slot's
  // row and weight are fetched with cross-lane shuffles.  Slots go in groups
  // of 8 whose loads are all issued before the first is added, so that 8 KiB
  // per wavefront are in flight; the sum still runs in slot order.
  for (int c0 = 0; c0 < H; c0 += kWave * 4) {
    const int base = c0 + lane * 4;
    const bool inside = base < H;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    bool started = false;
    for (int s0 = 0; s0 < k; s0 += 8) {
      float4 v[8];
      float wv[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sl = s0 + u;                       // < 40: a lane index
        const int row = __shfl(my_row, sl, kWave);
        wv[u] = __shfl(my_w, sl, kWave);
        ok[u] = sl < k && row >= 0 && row < T * k && inside;   // rows of d: T * k
        v[u] = ok[u] ? *reinterpret_cast<const float4*>(d + (int64_t)row * H + base)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!ok[u]) continue;
        float4 x = v[u];
        if (topk_w) { x.x = wv[u] * x.x; x.y = wv[u] * x.y; x.z = wv[u] * x.z; x.w = wv[u] * x.w; }
        if (started) { acc.x = acc.x + x.x; acc.y = acc.y + x.y; acc.z = acc.z + x.z; acc.w = acc.w + x.w; }
        else { acc = x; started = true; }
      }
    }
    if (!inside) continue;
    uint2 o;
    o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(y + t * (int64_t)H + base) = o;
  }
}

// The same sum for rows of H = 256 NC elements, slot by slot: lane l holds
// columns 4l + 256c (c < NC) of the token's sum, and each routed row is read
// whole (NC loads of 1 KiB per wavefront, one after another) before the next
// slot's, so a row's DRAM pages are read in one go.  The loads of G = 16 / NC
// slots are issued before the first of them is added (16 loads of 16 bytes per
// lane in flight); the sum runs in slot order with the same products and sums
// as unpermute_combine_kernel, so the results are identical.
template <int NC>
__global__ __launch_bounds__(256) void unpermute_combine_rows_kernel(
    const float* __restrict__ d, int64_t T, int k, const int32_t* __restrict__ tk_to_row,
    const float* __restrict__ topk_w, uint16_t* __restrict__ y) {
  constexpr int H = 256 * NC;
  constexpr int G = NC >= 16 ? 1 : 16 / NC;      // slots per group
  const int64_t t = (int64_t)blockIdx.x * kRows + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const int my_row = lane < k ? tk_to_row[t * k + lane] : -1;
  const float my_w = (lane < k && topk_w) ? topk_w[t * k + lane] : 1.0f;
  float4 acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  bool started = false;
  for (int s0 = 0; s0 < k; s0 += G) {
    float4 v[G][NC];
    float wv[G];
    bool ok[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int sl = s0 + u;                         // < 48: a lane index
      const int row = __shfl(my_row, sl, kWave);
      wv[u] = __shfl(my_w, sl, kWave);
      ok[u] = sl < k && row >= 0 && row < T * k;     // rows of d: T * k
      const float* src = d + (int64_t)(ok[u] ? row : 0) * H + 4 * lane;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        v[u][c] = ok[u] ? *reinterpret_cast<const float4*>(src + 256 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (!ok[u]) continue;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float4 x = v[u][c];
        if (topk_w) { x.x = wv[u] * x.x; x.y = wv[u] * x.y; x.z = wv[u] * x.z; x.w = wv[u] * x.w; }
        if (started) {
          acc[c].x = acc[c].x + x.x; acc[c].y = acc[c].y + x.y; acc[c].z = acc[c].z + x.z; acc[c].w = acc[c].w + x.w;
        } else {
          acc[c] = x;
        }
      }
      started = true;
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    uint2 o;
    o.x = f32_to_bf16_rne(acc[c].x) | (f32_to_bf16_rne(acc[c].y) << 16);
    o.y = f32_to_bf16_rne(acc[c].z) | (f32_to_bf16_rne(acc[c].w) << 16);
    *reinterpret_cast<uint2*>(y + t * (int64_t)H + 256 * c + 4 * lane) = o;
  }
}

// out[r] = x[row_to_tk[r] / k] for every routed row r.
__global__ __launch_bounds__(256) void permute_gather_kernel(
    const uint16_t* __restrict__ x, int64_t T, int H, int k, const int32_t* __restrict__ offsets, int E,
    const int32_t* __restrict__ row_to_tk, uint16_t* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * kRows + (threadIdx.x >> 6);
  if (r >= offsets[E] || r >= T * k) return;
  const int64_t t = min(max((int64_t)(row_to_tk[r] / k), (int64_t)0), T - 1);   // a bad map entry stays in x
  const uint16_t* src = x + t * (int64_t)H;
  uint16_t* dst = out + r * (int64_t)H;
  for (int base = lane_id() * 8; base < H; base += kWave * 8)
    *reinterpret_cast<uint4*>(dst + base) = *reinterpret_cast<const uint4*>(src + base);
}

// Gradient of h = w * silu(g) * u in float64 (sigmoid_f64, within 2^-50 of the
// sigmoid; silu = g * sigmoid), each output rounded once to bf16.
__global__ __launch_bounds__(256) void swiglu_backward_kernel(
    const float* __restrict__ gu, const float* __restrict__ dh, int64_t R_cap, int I,
    const int32_t* __restrict__ offsets, int E, const float* __restrict__ topk_w,
    const int32_t* __restrict__ row_to_tk, uint16_t* __restrict__ dgu) {
  __shared__ double exp2_tab[64];
  stage_exp2_table(exp2_tab);
  const int64_t r = (int64_t)blockIdx.x * kRows + (threadIdx.x >> 6);
  if (r >= offsets[E] || r >= R_cap) return;
  float w = 1.0f;
  if (topk_w) {   // the router weight of the row's (token, slot); a bad map entry gives 0
    const int32_t i = row_to_tk[r];
    w = (i >= 0 && i < R_cap) ? topk_w[i] : 0.0f;
  }
  const float* grow = gu + r * (int64_t)(2 * I);
  const float* drow = dh + r * (int64_t)I;
  uint16_t* orow = dgu + r * (int64_t)(2 * I);
  // 4 elements per lane per step (256 per wavefront), so that a row of any
  // multiple of 256 keeps every lane busy in the float64 work
  for (int base = lane_id() * 4; base < I; base += kWave * 4) {
    float gs[4], us[4], ds[4];
    *reinterpret_cast<float4*>(gs) = *reinterpret_cast<const float4*>(grow + base);
    *reinterpret_cast<float4*>(us) = *reinterpret_cast<const float4*>(grow + I + base);
    *reinterpret_cast<float4*>(ds) = *reinterpret_cast<const float4*>(drow + base);
    uint32_t og[2], ou[2];
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      uint32_t bg[2], bu[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const double g = gs[j + q], u = us[j + q];
        double t = ds[j + q];
        if (topk_w) t = t * (double)w;
        const double sig = sigmoid_f64(gs[j + q], exp2_tab);
        const double silu = g * sig;
        const double du = t * silu;
        const double dg = (t * u) * (sig * (1.0 + g * (1.0 - sig)));
        bg[q] = f64_to_bf16_rne(dg);
        bu[q] = f64_to_bf16_rne(du);
      }
      og[j / 2] = bg[0] | (bg[1] << 16);
      ou[j / 2] = bu[0] | (bu[1] << 16);
    }
    *reinterpret_cast<uint2*>(orow + base) = make_uint2(og[0], og[1]);
    *reinterpret_cast<uint2*>(orow + I + base) = make_uint2(ou[0], ou[1]);
  }
}

// out[b][j][i] = in[b][i][j] for a batch of bf16 matrices: 64 x 64 tiles
// through LDS, 16-byte loads and stores (rows and columns multiples of 8).
// Weight preparation for the NVFP4 input-gradient GEMM, which contracts a
// forward weight over its output dimension and so quantises its transpose.
constexpr int kTr = 64;
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             int rows, int cols,
                                                             uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[kTr][kTr + 2];
  const int64_t mat = (int64_t)rows * cols * blockIdx.z;
  const int r0 = blockIdx.y * kTr, c0 = blockIdx.x * kTr;
  for (int q = threadIdx.x; q < kTr * 8; q += 256) {
    const int r = q >> 3, ch = q & 7;
    if (r0 + r < rows && c0 + 8 * ch < cols) {
      const uint4 v = *reinterpret_cast<const uint4*>(in + mat + (int64_t)(r0 + r) * cols + c0 + 8 * ch);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[r][8 * ch + j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTr * 8; q += 256) {
    const int c = q >> 3, ch = q & 7;
    if (c0 + c < cols && r0 + 8 * ch < rows) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)tile[8 * ch + 2 * j][c] | ((uint32_t)tile[8 * ch + 2 * j + 1][c] << 16);
      *reinterpret_cast<uint4*>(out + mat + (int64_t)(c0 + c) * rows + r0 + 8 * ch) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" {

NVFP4MOE_API int unpermute_combine(const float* d, int64_t T, int32_t k, int64_t H,
                                   const int32_t* tk_to_row, const float* topk_w, uint16_t* y,
                                   void* stream) {
  if (T < 0 || k < 1 || k > NVFP4MOE_MAX_TOPK || H <= 0 || H % 8 != 0 || H > INT32_MAX / 2)
    return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  if (!d || !tk_to_row || !y) return NVFP4_ERR_NULL;
  if (!aligned16(d) || !aligned16(y)) return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)((T + kRows - 1) / kRows);
  if (H == 1024) unpermute_combine_rows_kernel<4><<<grid, 256, 0, s>>>(d, T, k, tk_to_row, topk_w, y);
  else if (H == 2048) unpermute_combine_rows_kernel<8><<<grid, 256, 0, s>>>(d, T, k, tk_to_row, topk_w, y);
  else if (H == 4096) unpermute_combine_rows_kernel<16><<<grid, 256, 0, s>>>(d, T, k, tk_to_row, topk_w, y);
  else unpermute_combine_kernel<<<grid, 256, 0, s>>>(d, T, k, (int)H, tk_to_row, topk_w, y);
  return launch_status();
}

NVFP4MOE_API int permute_gather_bf16(const uint16_t* x, int64_t T, int64_t H, int32_t k,
                                     const int32_t* expert_offsets, int32_t E,
                                     const int32_t* row_to_tk, uint16_t* out, void* stream) {
  if (T < 0 || k < 1 || k > NVFP4MOE_MAX_TOPK || H <= 0 || H % 8 != 0 || H > INT32_MAX / 2)
    return NVFP4_ERR_SHAPE;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS) return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  if (!x || !expert_offsets || !row_to_tk || !out) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t R_cap = T * k;
  permute_gather_kernel<<<(unsigned)((R_cap + kRows - 1) / kRows), 256, 0, s>>>(
      x, T, (int)H, k, expert_offsets, E, row_to_tk, out);
  return launch_status();
}

NVFP4MOE_API int swiglu_backward(const float* gu, const float* dh, int64_t R_cap, int64_t I,
                                 const int32_t* expert_offsets, int32_t E, const float* topk_w,
                                 const int32_t* row_to_tk, uint16_t* dgu, void* stream) {
  if (R_cap < 0 || I <= 0 || I % 8 != 0 || I > INT32_MAX / 4) return NVFP4_ERR_SHAPE;
  if (E < 1 || E > NVFP4MOE_MAX_EXPERTS) return NVFP4_ERR_SHAPE;
  if (R_cap == 0) return NVFP4_OK;
  if (!gu || !dh || !expert_offsets || !dgu) return NVFP4_ERR_NULL;
  if (topk_w && !row_to_tk) return NVFP4_ERR_NULL;
  if (!aligned16(gu) || !aligned16(dh) || !aligned16(dgu)) return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  swiglu_backward_kernel<<<(unsigned)((R_cap + kRows - 1) / kRows), 256, 0, s>>>(
      gu, dh, R_cap, (int)I, expert_offsets, E, topk_w, row_to_tk, dgu);
  return launch_status();
}

NVFP4MOE_API int bf16_transpose(const uint16_t* in, int64_t batches, int64_t rows, int64_t cols,
                                uint16_t* out, void* stream) {
  if (batches < 0 || batches > 65535 || rows < 0 || cols < 0 || rows % 8 != 0 || cols % 8 != 0)
    return NVFP4_ERR_SHAPE;
  if (rows > (int64_t)kTr * 65535 || cols > (int64_t)kTr * 65535 || rows * cols > INT32_MAX)
    return NVFP4_ERR_SHAPE;
  if (batches == 0 || rows == 0 || cols == 0) return NVFP4_OK;
  if (!in || !out) return NVFP4_ERR_NULL;
  if (!aligned16(in) || !aligned16(out)) return NVFP4_ERR_ALIGN;
  if (in == out) return NVFP4_ERR_ARG;
  const dim3 grid((unsigned)((cols + kTr - 1) / kTr), (unsigned)((rows + kTr - 1) / kTr), (unsigned)batches);
  transpose_bf16_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(in, (int)rows, (int)cols, out);
  return launch_status();
}

}  // extern "C"
