// Measurement helpers: the dense bf16 MFMA rate and the LDS read bandwidth the GPU sustains under
// full load, against which the attention kernels' rates are reported beside the published peaks.
// The MFMA probe runs four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave on
// register operands (no memory traffic inside the loop); the LDS probe issues 16-byte reads
// (the width of the kernels' operand reads) at consecutive addresses, so no bank conflicts.
// Each writes one value per lane so the work cannot be dropped.
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

// 64 KiB of LDS per workgroup, so two workgroups (eight waves) share a CU.  Each wave reads
// 16 KiB per iteration: sixteen 16-byte reads per lane, at an offset that changes with the
// iteration so the reads cannot be moved out of the loop.  Every address stays below 40 KiB.
constexpr int kLdsProbeInts = 16384;

__global__ __launch_bounds__(kProbeThreads) void lds_read_kernel(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) int buf[kLdsProbeInts];
  for (int i = threadIdx.x; i < kLdsProbeInts; i += kProbeThreads) buf[i] = (int)(i * 2654435761u);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int it = 0; it < iters; ++it) {
    int base = (it & 3) * 8192 + lane * 16;
    asm volatile("" : "+v"(base));
    const char* p = reinterpret_cast<const char*>(buf) + base;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(p + k * 1024);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = __builtin_bit_cast(float, acc);
}

hipError_t launch_lds_read(float* out, int n_workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(lds_read_kernel, dim3(n_workgroups), dim3(kProbeThreads), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace fa
