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
//
// An LDS bank probe: one wave per workgroup repeats one LDS access form at a
// per-lane byte offset (lanes with a negative offset stay inactive).  Read
// under rocprofv3 (SQ_LDS_BANK_CONFLICT), the probes give which lanes the LDS
// serves together for each access form and how many banks it spreads them
// over, the model the kernels' LDS layouts are designed against.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

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

// LDS access forms of the probe (kda_calibrate_lds `form`).  Each access is
// written with its own wait, so nothing is left in flight.
enum LdsForm : int {
  kRdB32 = 0, kRdB64 = 1, kRdB128 = 2, kRd2B64 = 3, kRd2B32 = 4,
  kWrB32 = 5, kWrB64 = 6, kWrB128 = 7, kWr2B32 = 8, kNumForms = 9
};
constexpr int kLdsBytes = 65536;
constexpr int kLdsSpan = 320;  // bytes an access may reach past its offset (the two-address forms)

struct LaneOffsets {
  int off[64];
};

template <int FORM>
__global__ __launch_bounds__(64) void lds_probe(LaneOffsets lo, int iters, float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) float lds[kLdsBytes / 4];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += 64) lds[i] = static_cast<float>(i & 1023);
  __syncthreads();
  const int lane = threadIdx.x;
  const int off = lo.off[lane];
  float acc = 0.f;
  if (off >= 0) {
    const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + static_cast<uint32_t>(off);
    f32x4 w = {1.f, 2.f, 3.f, 4.f};
    for (int it = 0; it < iters; ++it) {
      if constexpr (FORM == kRdB32) {
        float v;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
        acc += v;
      } else if constexpr (FORM == kRdB64) {
        float __attribute__((ext_vector_type(2))) v;
        asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
        acc += v[0] + v[1];
      } else if constexpr (FORM == kRdB128) {
        f32x4 v;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
        acc += v[0] + v[3];
      } else if constexpr (FORM == kRd2B64) {  // two 8-byte reads, 32 bytes apart
        f32x4 v;
        asm volatile("ds_read2_b64 %0, %1 offset1:4\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
        acc += v[0] + v[3];
      } else if constexpr (FORM == kRd2B32) {  // two 4-byte reads, 16 bytes apart
        float __attribute__((ext_vector_type(2))) v;
        asm volatile("ds_read2_b32 %0, %1 offset1:4\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
        acc += v[0] + v[1];
      } else if constexpr (FORM == kWrB32) {
        asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(a), "v"(w[0]) : "memory");
        w[0] += 1.f;
      } else if constexpr (FORM == kWrB64) {
        const float __attribute__((ext_vector_type(2))) x = {w[0], w[1]};
        asm volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(a), "v"(x) : "memory");
        w[0] += 1.f;
      } else if constexpr (FORM == kWrB128) {
        asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(a), "v"(w) : "memory");
        w[0] += 1.f;
      } else {  // kWr2B32: two 4-byte writes, 272 bytes apart
        asm volatile("ds_write2_b32 %0, %1, %1 offset1:68\n\ts_waitcnt lgkmcnt(0)" : : "v"(a), "v"(w[0]) : "memory");
        w[0] += 1.f;
      }
    }
    acc += w[0];
  }
  sink[static_cast<long>(blockIdx.x) * 64 + lane] = acc;
}

template <int... F>
constexpr void (*lds_probes(int f, std::integer_sequence<int, F...>))(LaneOffsets, int, float*) {
  void (*fns[])(LaneOffsets, int, float*) = {&lds_probe<F>...};
  return fns[f];
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

int kda_calibrate_lds(int form, const int* lane_offsets, int blocks, int iters, float* sink, void* stream) {
  if (form < 0 || form >= kNumForms || lane_offsets == nullptr || blocks < 1 || iters < 1 || sink == nullptr)
    return 1;
  LaneOffsets lo;
  for (int l = 0; l < 64; ++l) {
    const int o = lane_offsets[l];
    if (o >= kLdsBytes - kLdsSpan || (o >= 0 && o % 4 != 0)) return 1;  // in bounds, 4-byte aligned
    lo.off[l] = o < 0 ? -1 : o;
  }
  const auto fn = lds_probes(form, std::make_integer_sequence<int, kNumForms>{});
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(64), 0, static_cast<hipStream_t>(stream), lo, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
