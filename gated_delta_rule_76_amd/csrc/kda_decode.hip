// T = 1 decode step of Kimi Delta Attention on gfx950.
//
// Per (batch, head), with the fp32 state S (d_k x d_v) updated in place
// (page "Yanjiu KimiK3 ...", http://www.pwwt.cn/news/3763336/, section 4 KDA
// update; section 3 prediction and error; section 2.1 readout):
//   S' = Diag(alpha) S             decay every key channel (row of S)
//   v_hat = S'^T k, z = S'^T q     two reductions over d_k, same pass over S
//   u = beta (v - v_hat)           the delta rule's scaled prediction error
//                                  (u = beta v without the correction)
//   S <- S' + k u^T                written back in place
//   o = z + (k^T q) u              = S_new^T q, no second pass over S
//
// The gate is one decay per key channel (KDA), one per head broadcast over the
// channels (Gated DeltaNet), or none.  With the fused prologue the inputs are
// raw projections: q and k are L2-normalised, alpha = exp(-c softplus(g)),
// beta = sigmoid(b), all in fp32 inside the kernel.
//
// The kernel is bound by HBM: it reads and writes each state once.  One
// workgroup owns one head.  Thread t holds a float4 column group (4 adjacent
// value columns) for every RG-th key row, so each load instruction of a wave
// touches whole contiguous state rows (fully coalesced 16-byte accesses).
// The state for the thread's rows stays in registers between the reduction
// and the write-back.  Global indices go through chk() / chk_ok()
// (kda_check.h): checked in the checked build, free in the normal one.
#include "kda_check.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// Check sites of this unit (bits of the checked build's failure mask, before
// the unit's shift).
enum : int { kSiteState = 0, kSiteQKA = 1, kSiteV = 2, kSiteBeta = 3, kSiteOut = 4 };

template <int DK, int DV>
struct DecodeShape {
  static constexpr int CG = DV / 4;                              // float4 column groups
  static constexpr int NTH = (DK * CG < 512) ? DK * CG : 512;    // threads per workgroup
  static constexpr int RG = NTH / CG;                            // row groups
  static constexpr int RPT = DK / RG;                            // rows per thread
  static constexpr int NW = NTH / 64;                            // waves
  static_assert(NTH % 64 == 0 && RPT >= 1 && CG <= 64, "decode shape");
};

// PLAIN: the KDA step itself (per-channel gate, delta rule, inputs as given),
// compiled without the variant branches; the general kernel reads gate, rule
// and fused at run time.
template <typename E, int DK, int DV, bool PLAIN>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NTH)) void decode_kernel(
    const typename E::storage* __restrict__ q, const typename E::storage* __restrict__ k,
    const typename E::storage* __restrict__ v, const typename E::storage* __restrict__ alpha,
    const typename E::storage* __restrict__ beta, float* __restrict__ S,
    typename E::storage* __restrict__ o, int gate, int rule, int fused, float gscale) {
  using Sh = DecodeShape<DK, DV>;
  if constexpr (PLAIN) {
    gate = kGateChannel;
    rule = kRuleDelta;
    fused = 0;
  }
  const long head = blockIdx.x;  // b * H + h
  const int tid = threadIdx.x;
  const int cg = tid % Sh::CG;
  const int rg = tid / Sh::CG;

  float4* __restrict__ S4 = reinterpret_cast<float4*>(S + head * DK * DV);
  // extents for the checked build (B * H = gridDim.x heads)
  const long nhead = gridDim.x, ns4 = DK * DV / 4;

  // Issue the state loads first: they are the long-latency part.
  float4 s[Sh::RPT];
#pragma unroll
  for (int m = 0; m < Sh::RPT; ++m) s[m] = S4[chk((rg + Sh::RG * m) * Sh::CG + cg, ns4, kSiteState)];

  __shared__ float sq[DK], sk[DK], sa[DK], sv[DV];
  // per-wave partial reductions, one float4 per column group (16-byte
  // accesses: one LDS write per lane, no bank conflicts)
  __shared__ float4 red_y[Sh::NW][Sh::CG], red_z[Sh::NW][Sh::CG];
  __shared__ float red_kq[Sh::NW];
  // gate: one decay per channel, one per head (broadcast), or none; with the
  // fused prologue the gate and beta arrive as raw projections
  float ah = gate == kGateHead ? load_scalar(alpha, chk(head, nhead, kSiteQKA)) : 1.f;
  if (fused && gate == kGateHead) ah = gate_map(ah, gscale);
  for (int i = tid; i < DK; i += Sh::NTH) {
    sq[i] = load_scalar(q, chk(head * DK + i, nhead * DK, kSiteQKA));
    sk[i] = load_scalar(k, chk(head * DK + i, nhead * DK, kSiteQKA));
    float a = ah;
    if (gate == kGateChannel) {
      a = load_scalar(alpha, chk(head * DK + i, nhead * DK, kSiteQKA));
      if (fused) a = gate_map(a, gscale);
    }
    sa[i] = a;
  }
  for (int j = tid; j < DV; j += Sh::NTH) sv[j] = load_scalar(v, chk(head * DV + j, nhead * DV, kSiteV));
  float bt = load_scalar(beta, chk(head, nhead, kSiteBeta));
  if (fused) bt = sigmoid_f(bt);
  __syncthreads();
  if (fused) {  // L2-normalise q and k: wave 0 reduces, everyone rescales
    __shared__ float inv[2];
    if (tid < 64) {
      float ssq = 0.f, ssk = 0.f;
      for (int i = tid; i < DK; i += 64) { ssq += sq[i] * sq[i]; ssk += sk[i] * sk[i]; }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) { ssq += __shfl_xor(ssq, off); ssk += __shfl_xor(ssk, off); }
      if (tid == 0) {
        inv[0] = ssq > 0.f ? rsqrtf(ssq) : 0.f;
        inv[1] = ssk > 0.f ? rsqrtf(ssk) : 0.f;
      }
    }
    __syncthreads();
    const float iq = inv[0], ik = inv[1];
    for (int i = tid; i < DK; i += Sh::NTH) { sq[i] *= iq; sk[i] *= ik; }
    __syncthreads();
  }

  float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
  float z0 = 0.f, z1 = 0.f, z2 = 0.f, z3 = 0.f;
  float kq = 0.f;
#pragma unroll
  for (int m = 0; m < Sh::RPT; ++m) {
    const int i = rg + Sh::RG * m;
    const float a = sa[i], ki = sk[i], qi = sq[i];
    s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
    y0 += ki * s[m].x; y1 += ki * s[m].y; y2 += ki * s[m].z; y3 += ki * s[m].w;
    z0 += qi * s[m].x; z1 += qi * s[m].y; z2 += qi * s[m].z; z3 += qi * s[m].w;
    kq += ki * qi;
  }
  // Reduce over the row groups inside the wave (lanes with equal cg).
#pragma unroll
  for (int off = Sh::CG; off < 64; off <<= 1) {
    y0 += __shfl_xor(y0, off); y1 += __shfl_xor(y1, off);
    y2 += __shfl_xor(y2, off); y3 += __shfl_xor(y3, off);
    z0 += __shfl_xor(z0, off); z1 += __shfl_xor(z1, off);
    z2 += __shfl_xor(z2, off); z3 += __shfl_xor(z3, off);
    kq += __shfl_xor(kq, off);
  }
  if constexpr (Sh::NW > 1) {
    const int lane = tid & 63, w = tid >> 6;
    if (lane < Sh::CG) {
      red_y[w][cg] = float4{y0, y1, y2, y3};
      red_z[w][cg] = float4{z0, z1, z2, z3};
      if (cg == 0) red_kq[w] = kq;
    }
    __syncthreads();
    y0 = y1 = y2 = y3 = z0 = z1 = z2 = z3 = kq = 0.f;
#pragma unroll
    for (int ww = 0; ww < Sh::NW; ++ww) {
      const float4 ry = red_y[ww][cg], rz = red_z[ww][cg];
      y0 += ry.x; y1 += ry.y; y2 += ry.z; y3 += ry.w;
      z0 += rz.x; z1 += rz.y; z2 += rz.z; z3 += rz.w;
      kq += red_kq[ww];
    }
  }
  if (rule == kRuleLinear) y0 = y1 = y2 = y3 = 0.f;  // no correction: u = beta v
  const float u0 = bt * (sv[4 * cg + 0] - y0), u1 = bt * (sv[4 * cg + 1] - y1);
  const float u2 = bt * (sv[4 * cg + 2] - y2), u3 = bt * (sv[4 * cg + 3] - y3);
  if (rg == 0 && chk_ok(head * DV + 4 * cg, nhead * DV, kSiteOut, 4)) {
    const long ob = head * DV + 4 * cg;
    store_scalar(o, ob + 0, z0 + kq * u0);
    store_scalar(o, ob + 1, z1 + kq * u1);
    store_scalar(o, ob + 2, z2 + kq * u2);
    store_scalar(o, ob + 3, z3 + kq * u3);
  }
#pragma unroll
  for (int m = 0; m < Sh::RPT; ++m) {
    const int i = rg + Sh::RG * m;
    const float ki = sk[i];
    s[m].x += ki * u0; s[m].y += ki * u1; s[m].z += ki * u2; s[m].w += ki * u3;
    if (chk_ok(i * Sh::CG + cg, ns4, kSiteState)) S4[i * Sh::CG + cg] = s[m];
  }
}

template <typename E, int DK, int DV>
hipError_t launch_decode_t(const DecodeArgs& a) {
  using Sh = DecodeShape<DK, DV>;
  using St = typename E::storage;
  const bool plain = a.gate == kGateChannel && a.rule == kRuleDelta && !a.fused;
  auto kern = plain ? decode_kernel<E, DK, DV, true> : decode_kernel<E, DK, DV, false>;
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(Sh::NTH), 0, a.stream,
                     static_cast<const St*>(a.q), static_cast<const St*>(a.k),
                     static_cast<const St*>(a.v), static_cast<const St*>(a.alpha),
                     static_cast<const St*>(a.beta), a.S, static_cast<St*>(a.o), a.gate, a.rule,
                     a.fused ? 1 : 0, a.gate_scale);
  return hipGetLastError();
}

template <typename E, int DK>
hipError_t dispatch_dv(const DecodeArgs& a) {
  switch (a.d_v) {
    case 16: return launch_decode_t<E, DK, 16>(a);
    case 32: return launch_decode_t<E, DK, 32>(a);
    case 64: return launch_decode_t<E, DK, 64>(a);
    case 128: return launch_decode_t<E, DK, 128>(a);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t dispatch_dk(const DecodeArgs& a) {
  switch (a.d_k) {
    case 16: return dispatch_dv<E, 16>(a);
    case 32: return dispatch_dv<E, 32>(a);
    case 64: return dispatch_dv<E, 64>(a);
    case 128: return dispatch_dv<E, 128>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
  return a.bf16 ? dispatch_dk<Bf16>(a) : dispatch_dk<F32>(a);
}

unsigned decode_check_take() { return check_take(); }

}  // namespace kda
