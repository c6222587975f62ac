// Measurement helper: the dense bf16 MFMA rate the GPU sustains under full load, against which
// the attention kernels' rates are reported beside the published peak.  Each wave runs four
// independent accumulator chains of v_mfma_f32_32x32x16_bf16 on register operands (no memory
// traffic inside the loop) and writes one value per lane so the work cannot be dropped.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void mfma_peak_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  e16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((lane + i) & 3);
    b[i] = (__bf16)(float)((lane + 2 * i) & 3);
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 32; ++m) acc[m & 3] = mfma32x32x16<kElemBf16>(a, b, acc[m & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

hipError_t launch_mfma_peak(float* out, int n_workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(n_workgroups), dim3(kProbeThreads), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace fa
