// Measurement aid: the practical FP16 MFMA rate of the device.
//
// Every wavefront issues back-to-back v_mfma_f32_32x32x16_f16 on register
// operands (8 independent accumulators, so no MFMA waits for another's
// result), two wavefronts per SIMD.  Nothing is loaded; the sums leave through
// one store per thread at the end.  Divided into the FLOPs issued, the
// elapsed time gives the rate the matrix cores sustain at the clock the
// device runs under full MFMA load, next to the nominal peak.
#include "common.h"

namespace nvfp4moe {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kCeilWaves = 8;
constexpr int kCeilGrid = 256;

__global__ __launch_bounds__(kCeilWaves * 64) void mfma_ceiling_kernel(int64_t iters, float* sink) {
  floatx16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = floatx16{};
  const half8 a = (half8)(_Float16)(threadIdx.x * 1e-3f);
  const half8 b0 = (half8)(_Float16)1e-3f, b1 = (half8)(_Float16)2e-3f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16((i & 1) ? b1 : b0, a, acc[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][15];
  sink[blockIdx.x * (kCeilWaves * 64) + threadIdx.x] = s;
}

}  // namespace
}  // namespace nvfp4moe

using namespace nvfp4moe;

extern "C" NVFP4MOE_API int nvfp4moe_mfma_ceiling(int64_t iters, float* sink, void* stream) {
  if (iters < 1 || iters > 10000000) return NVFP4_ERR_SHAPE;
  if (!sink) return NVFP4_ERR_NULL;
  if (!aligned16(sink)) return NVFP4_ERR_ALIGN;
  mfma_ceiling_kernel<<<kCeilGrid, kCeilWaves * 64, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return launch_status();
}
