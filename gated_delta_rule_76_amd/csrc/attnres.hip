// AttnRes depth aggregation on gfx950 (page "Yanjiu KimiK3 ...",
// http://www.pwwt.cn/news/3763336/, section 8):
//   out[n] = sum_i softmax_i(q[n] . k[i, n]) h[i, n],  i over the L earlier layers.
//
// HBM-bound: every token reads L rows of h (L * d elements) and writes one
// row.  One workgroup per token:
//   1. scores: wave w takes layers w, w + 4, ...; lanes split d_k, a
//      shuffle reduction gives q . k_i, kept in LDS
//   2. softmax: wave 0 takes the max and the sum over the L scores (fp32,
//      max-subtracted) and leaves the weights in LDS
//   3. weighted sum: each thread owns two groups of 8 adjacent columns per
//      sweep of d and walks the layers four at a time (eight 16-byte row
//      loads in flight, streaming), accumulating in fp32
// Global indices go through chk() / chk_ok() (kda_check.h): checked in the
// checked build, free in the normal one.
#include <math.h>
#include <stdint.h>

#include "../../include/attnres.h"
#include "kda_check.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLayers = 1024;

// Check sites of this unit (bits of the checked build's failure mask, before
// the unit's shift).
enum : int { kSiteQ = 0, kSiteK = 1, kSiteH = 2, kSiteOut = 3 };

// The layer outputs are read once per call: streaming (nontemporal) loads
// keep them from displacing other lines in the caches.
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));

template <typename St>
struct Vec8;
template <>
struct Vec8<uint16_t> {  // 8 bf16 = 16 bytes
  uint4 r;
  __device__ __forceinline__ void load(const uint16_t* p) {
    const u32x4_nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    r = uint4{t[0], t[1], t[2], t[3]};
  }
  __device__ __forceinline__ void fma(float w, float* acc) const {
    acc[0] += w * __uint_as_float(r.x << 16); acc[1] += w * __uint_as_float(r.x & 0xffff0000u);
    acc[2] += w * __uint_as_float(r.y << 16); acc[3] += w * __uint_as_float(r.y & 0xffff0000u);
    acc[4] += w * __uint_as_float(r.z << 16); acc[5] += w * __uint_as_float(r.z & 0xffff0000u);
    acc[6] += w * __uint_as_float(r.w << 16); acc[7] += w * __uint_as_float(r.w & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* acc) {
    uint4 o;
    o.x = f32_to_bf16_bits(acc[0]) | (static_cast<unsigned>(f32_to_bf16_bits(acc[1])) << 16);
    o.y = f32_to_bf16_bits(acc[2]) | (static_cast<unsigned>(f32_to_bf16_bits(acc[3])) << 16);
    o.z = f32_to_bf16_bits(acc[4]) | (static_cast<unsigned>(f32_to_bf16_bits(acc[5])) << 16);
    o.w = f32_to_bf16_bits(acc[6]) | (static_cast<unsigned>(f32_to_bf16_bits(acc[7])) << 16);
    *reinterpret_cast<uint4*>(p) = o;
  }
};
template <>
struct Vec8<float> {  // 8 fp32 = 32 bytes
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    const f32x4_nt x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p));
    const f32x4_nt y = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p + 4));
    a = float4{x[0], x[1], x[2], x[3]};
    b = float4{y[0], y[1], y[2], y[3]};
  }
  __device__ __forceinline__ void fma(float w, float* acc) const {
    acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
    acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* acc) {
    *reinterpret_cast<float4*>(p) = float4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<float4*>(p + 4) = float4{acc[4], acc[5], acc[6], acc[7]};
  }
};

template <typename E>
__global__ __launch_bounds__(kThreads) void attnres_kernel(
    const typename E::storage* __restrict__ q, const typename E::storage* __restrict__ k,
    const typename E::storage* __restrict__ h, typename E::storage* __restrict__ out, int L,
    int N, int dk, int d) {
  using St = typename E::storage;
  __shared__ float w[kMaxLayers];
  __shared__ float red[2];
  const long n = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // extents for the checked build
  const long nq = static_cast<long>(N) * dk, nk = nq * L, nh = static_cast<long>(L) * N * d;
  const long no = static_cast<long>(N) * d;

  // 1. scores q . k_i
  for (int i = wave; i < L; i += kThreads / 64) {
    const long ki = (static_cast<long>(i) * N + n) * dk;
    float s = 0.f;
    for (int c = lane; c < dk; c += 64)
      s += load_scalar(q, chk(n * dk + c, nq, kSiteQ)) * load_scalar(k, chk(ki + c, nk, kSiteK));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) w[i] = s;
  }
  __syncthreads();
  // 2. softmax over the layers
  if (wave == 0) {
    float m = -INFINITY;
    for (int i = lane; i < L; i += 64) m = fmaxf(m, w[i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float z = 0.f;
    for (int i = lane; i < L; i += 64) {
      const float e = expf(w[i] - m);
      w[i] = e;
      z += e;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    if (lane == 0) red[0] = 1.f / z;
  }
  __syncthreads();
  const float inv = red[0];
  // 3. weighted sum of the layer outputs: two column groups per thread and
  //    four layers per step keep eight 16-byte loads in flight
  const long rowstride = static_cast<long>(N) * d;  // between layers
  const long hn = n * d;
  for (int c0 = 8 * tid; c0 < d; c0 += 16 * kThreads) {
    const int c1 = c0 + 8 * kThreads;
    const bool two = c1 < d;
    const int c1s = two ? c1 : c0;  // a valid column for the loads when there is no second group
    float a0[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float a1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int i = 0;
    for (; i + 4 <= L; i += 4) {
      Vec8<St> x[4], y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j].load(h + chk(hn + (i + j) * rowstride + c0, nh, kSiteH, 8));
        y[j].load(h + chk(hn + (i + j) * rowstride + c1s, nh, kSiteH, 8));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j].fma(w[i + j], a0);
        y[j].fma(w[i + j], a1);
      }
    }
    for (; i < L; ++i) {
      Vec8<St> x, y;
      x.load(h + chk(hn + i * rowstride + c0, nh, kSiteH, 8));
      y.load(h + chk(hn + i * rowstride + c1s, nh, kSiteH, 8));
      x.fma(w[i], a0);
      y.fma(w[i], a1);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) { a0[e] *= inv; a1[e] *= inv; }
    if (chk_ok(n * d + c0, no, kSiteOut, 8)) Vec8<St>::store(out + n * d + c0, a0);
    if (two && chk_ok(n * d + c1, no, kSiteOut, 8)) Vec8<St>::store(out + n * d + c1, a1);
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

}  // namespace

unsigned attnres_check_take() { return check_take(); }

}  // namespace kda

extern "C" int attnres_forward(const void* q, const void* k, const void* h, void* out, int L, int N,
                               int d_k, int d, int dtype, void* stream) {
  using namespace kda;
  try {
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
    if (!q || !k || !h || !out || N < 1 || L < 1 || d_k < 1 || d < 1) return KDA_ERR_INVALID_ARG;
    if (L > kMaxLayers || d_k > 512 || d % 8 != 0) return KDA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(h) || !aligned16(out)) return KDA_ERR_INVALID_ARG;
    const size_t esz = dtype == KDA_BF16 ? 2 : 4;
    const size_t nq = static_cast<size_t>(N) * d_k * esz, nk = nq * L;
    const size_t nh = static_cast<size_t>(L) * N * d * esz, no = static_cast<size_t>(N) * d * esz;
    if (overlaps(out, no, q, nq) || overlaps(out, no, k, nk) || overlaps(out, no, h, nh))
      return KDA_ERR_INVALID_ARG;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == KDA_BF16)
      hipLaunchKernelGGL(attnres_kernel<Bf16>, dim3(N), dim3(kThreads), 0, s,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(h), static_cast<uint16_t*>(out), L, N, d_k, d);
    else
      hipLaunchKernelGGL(attnres_kernel<F32>, dim3(N), dim3(kThreads), 0, s,
                         static_cast<const float*>(q), static_cast<const float*>(k),
                         static_cast<const float*>(h), static_cast<float*>(out), L, N, d_k, d);
    if (hipGetLastError() != hipSuccess) return KDA_ERR_HIP;
    return checked_finish(s, KDA_OK);
  } catch (...) {
    return KDA_ERR_HIP;
  }
}
