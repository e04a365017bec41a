// Matrix-core throughput probe: back-to-back bf16 matrix instructions on
// register operands, eight independent accumulator chains per wavefront so
// that no instruction waits on the one before it.  Its rate is the ceiling
// the matrix-core kernels' FLOP rates are read against (the published dense
// figure is the other).
#include "probes.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ sink, int iterations) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.125f * (float)((lane + k) & 7));
    b[k] = (__bf16)(0.0625f * (float)((lane * 3 + k) & 15));
  }
  f32x4_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iterations; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  if (s == -1.0f) sink[0] = s;              // never true (every product is >= 0): keeps the work
}

}  // namespace

hipError_t launch_mfma_peak(float* sink, int workgroups, int iterations, hipStream_t stream) {
  if (workgroups <= 0 || iterations <= 0) return hipSuccess;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, sink, iterations);
  return hipGetLastError();
}

}  // namespace pkv
