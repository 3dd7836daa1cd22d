// Calibration kernels for the benchmark (not part of the KDA library's C
// ABI): a dense bf16 matrix-core loop that measures the attainable MFMA rate
// of the device.  The benchmark divides the prefill's algorithmic flop rate
// by it, and profiles it under the same rocprofv3 counters as the KDA
// kernels, so that their MFMA-busy counts can be read against a kernel that
// keeps the matrix cores saturated.
//
// Each wave keeps NACC independent accumulators and issues one MFMA into each
// per iteration, so consecutive MFMAs never depend on each other; every CU
// runs eight workgroups of four waves (eight waves per SIMD).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "calibrate.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// 16x16x32 bf16 (16 384 flops per instruction)
__global__ __launch_bounds__(kThreads) void mfma16_loop(int iters, float* __restrict__ sink) {
  constexpr int NACC = 8;
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 0.001f * (lane + e));
    b[e] = static_cast<__bf16>(0.5f - 0.001f * (lane - e));
  }
  f32x4 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[static_cast<long>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

// 32x32x16 bf16 (32 768 flops per instruction)
__global__ __launch_bounds__(kThreads) void mfma32_loop(int iters, float* __restrict__ sink) {
  constexpr int NACC = 4;
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 0.001f * (lane + e));
    b[e] = static_cast<__bf16>(0.5f - 0.001f * (lane - e));
  }
  f32x16 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[static_cast<long>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int kda_calibrate_threads_per_block(void) { return kThreads; }

double kda_calibrate_flops(int kind, int blocks, int iters) {
  const double per_wave_iter = kind == 0 ? 8.0 * 16 * 16 * 32 * 2 : 4.0 * 32 * 32 * 16 * 2;
  return per_wave_iter * (kThreads / 64) * static_cast<double>(blocks) * iters;
}

int kda_calibrate_mfma(int kind, int blocks, int iters, float* sink, void* stream) {
  if ((kind != 0 && kind != 1) || blocks < 1 || iters < 1 || sink == nullptr) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(mfma16_loop, dim3(blocks), dim3(kThreads), 0, st, iters, sink);
  else
    hipLaunchKernelGGL(mfma32_loop, dim3(blocks), dim3(kThreads), 0, st, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
