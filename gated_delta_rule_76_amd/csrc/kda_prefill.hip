// Chunked (WY-form) prefill of Kimi Delta Attention on gfx950.
//
// The method (page "Yanjiu KimiK3 ...", http://www.pwwt.cn/news/3763336/):
// KDA update S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
// (section 4), readout o_t = S_t^T q_t (section 2.1).  Section 6 evaluates it
// chunk by chunk: the state passes between chunks of C tokens, and inside a
// chunk the C rank-one transitions are combined into "diagonal minus low
// rank" form so the work becomes a few matrix products (section 6.2).
//
// Per chunk, rows r = 0..C-1, gamma_r = prod_{s<=r} alpha_s per key channel:
//   K+ = K * gamma,  Q+ = Q * gamma,  K- = K / gamma,  Kbar = K- * gamma_C
//   A  = strict_lower(K+ K-^T)        (decayed key-key products)
//   P  = lower(Q+ K-^T)               (decayed query-key products, diagonal kept)
//   Tm = (I + Diag(beta) A)^{-1} Diag(beta)
//   U  = Tm (V - K+ S)                (the chunk's effective writes)
//   O  = Q+ S + P U
//   S <- Diag(gamma_C) S + Kbar^T U
// which unrolls the token recurrence exactly; the chunk's transition product
// is Diag(gamma_C) - Kbar^T Tm K+, the page's P = D - K W^T.
//
// Work split.  One workgroup (4 waves) owns one (batch, head, value block of
// DVB columns) and walks the chunks in order, so the fp32 state never leaves
// registers.  Each wave owns 16-column slabs of the state as 16x16 MFMA
// accumulator tiles.  Per chunk:
//   1. load alpha/k/q (16-byte loads), scan the per-channel cumulative decay
//      (in-thread over a row group, then across row groups through LDS) and
//      write the bf16 (or fp32) operand tiles K+, K-, Q+, Kbar^T into LDS;
//   2. MFMA the lower-triangular tiles of A and P;
//   3. invert the unit lower-triangular I + Diag(beta) A in fp32: 16x16
//      diagonal blocks by substitution (one wave per block), off-diagonal
//      blocks with fp32 MFMA, level by level;
//   4. each wave: X = K+ S, R = V - X, U = Tm R, O = Q+ S + P U, state update,
//      all as MFMA with the state and intermediate tiles converted from
//      accumulator registers straight into operand registers.
//
// MFMA operand convention.  A 16x16 tile product over a k range of 32 takes
// 8 values per lane; lane (g = lane/16, c = lane%16) holds row/column c and
// k indices {32s+4g+e, 32s+16+4g+e : e = 0..3}.  This is exactly what a lane
// holds of two vertically stacked accumulator tiles, so accumulators become
// operands without any data movement; LDS operands are read with the same
// index map (two 4-element reads).  The reduction does not depend on which k
// each (lane, element) slot carries as long as both operands agree.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int NTH = 256;
constexpr int NW = NTH / 64;

__device__ __forceinline__ f32x8 load8f(const uint16_t* p) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  f32x8 x;
  x[0] = __uint_as_float(r.x << 16); x[1] = __uint_as_float(r.x & 0xffff0000u);
  x[2] = __uint_as_float(r.y << 16); x[3] = __uint_as_float(r.y & 0xffff0000u);
  x[4] = __uint_as_float(r.z << 16); x[5] = __uint_as_float(r.z & 0xffff0000u);
  x[6] = __uint_as_float(r.w << 16); x[7] = __uint_as_float(r.w & 0xffff0000u);
  return x;
}
__device__ __forceinline__ f32x8 load8f(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Matrix-core operand traits: bf16 operands (one 16x16x32 MFMA per k-step)
// or fp32 operands (eight 16x16x4 fp32 MFMAs per k-step, same index map).
template <typename E>
struct Mma;

template <>
struct Mma<Bf16> {
  using lds_t = __bf16;
  using frag = bf16x8;
  static constexpr int PAD = 8;  // 16 bytes of row padding in LDS
  static __device__ __forceinline__ lds_t cvt(float x) { return static_cast<__bf16>(x); }
  static __device__ __forceinline__ frag pair(const lds_t* lo, const lds_t* hi) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(lo);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(hi);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ frag half(const lds_t* lo) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(lo);
    const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
    return __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ frag from_acc(f32x4 lo, f32x4 hi) {
    frag r;
    r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
    r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
    return r;
  }
  static __device__ __forceinline__ void store8(lds_t* p, f32x8 x) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x8*>(p) = r;
  }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<F32> {
  using lds_t = float;
  using frag = f32x8;
  static constexpr int PAD = 4;
  static __device__ __forceinline__ lds_t cvt(float x) { return x; }
  static __device__ __forceinline__ frag pair(const lds_t* lo, const lds_t* hi) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(lo);
    const f32x4 b = *reinterpret_cast<const f32x4*>(hi);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ frag half(const lds_t* lo) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(lo);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ frag from_acc(f32x4 lo, f32x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ void store8(lds_t* p, f32x8 x) {
    *reinterpret_cast<f32x4*>(p) = __builtin_shufflevector(x, x, 0, 1, 2, 3);
    *reinterpret_cast<f32x4*>(p + 4) = __builtin_shufflevector(x, x, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
};

template <typename E, int DK, int DVB, int C>
struct Cfg {
  using M = Mma<E>;
  using lds_t = typename M::lds_t;
  static constexpr int NT = C / 16;          // 16-row tiles per chunk
  static constexpr int NTK = DK / 16;        // 16-row tiles of the state
  static constexpr int NKS = (NTK + 1) / 2;  // 32-wide k-steps over d_k
  static constexpr bool KODD = (NTK & 1) != 0;
  static constexpr int NCS = (NT + 1) / 2;   // 32-wide k-steps over the chunk
  static constexpr bool CODD = (NT & 1) != 0;
  static constexpr int NSLAB = DVB / 16;     // 16-column state slabs
  static constexpr int SPW = (NSLAB + NW - 1) / NW;  // slabs per wave
  static constexpr int NCG = DK / 8;         // prologue: 8-channel groups
  static constexpr int NRG0 = NTH / NCG;
  static constexpr int NRG = NRG0 < C ? NRG0 : C;  // prologue row groups in use
  static constexpr int RPG = C / NRG;        // rows per prologue row group
  static constexpr int LDK = DK + M::PAD;    // row stride of C x DK tiles
  static constexpr int LDC = C + M::PAD;     // row stride of ? x C tiles
  static constexpr int LDF = C + 1;          // row stride of the fp32 C x C tiles
  static_assert(NRG * RPG == C && NCG * NRG <= NTH, "prologue map");

  struct Smem {
    alignas(16) lds_t Kp[C * LDK];
    alignas(16) lds_t Km[C * LDK];
    alignas(16) lds_t Qp[C * LDK];
    alignas(16) lds_t KbT[DK * LDC];
    alignas(16) lds_t Tm[C * LDC];
    alignas(16) lds_t P[C * LDC];
    alignas(16) float Mf[C * LDF];  // Diag(beta) A, strictly lower, fp32
    alignas(16) float Xf[C * LDF];  // (I + Diag(beta) A)^{-1}, fp32
    alignas(16) float gC[DK];
    alignas(16) float beta[C];
    alignas(16) float scan[NRG * DK];
  };
  static constexpr size_t smem_bytes = sizeof(Smem);
};

template <int DK, int DVB, int C>
constexpr bool fits_lds_bf16() { return Cfg<Bf16, DK, DVB, C>::smem_bytes <= 160 * 1024; }

template <typename E, int DK, int DVB, int C>
__global__ __launch_bounds__(NTH) void prefill_kernel(
    const typename E::storage* __restrict__ q, const typename E::storage* __restrict__ k,
    const typename E::storage* __restrict__ v, const typename E::storage* __restrict__ alpha,
    const typename E::storage* __restrict__ beta, const float* __restrict__ S0,
    typename E::storage* __restrict__ o, float* __restrict__ ST, int T, int H, int DV) {
  using K = Cfg<E, DK, DVB, C>;
  using M = typename K::M;
  using lds_t = typename K::lds_t;
  using frag = typename M::frag;
  __shared__ typename K::Smem sm;

  const int vb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const long bh = static_cast<long>(b) * H + h;
  auto tok = [&](int t) -> long { return (static_cast<long>(b) * T + t) * H + h; };

  // The strictly upper parts of Tm, P, Mf are never written per chunk: zero once.
  for (int i = tid; i < C * K::LDC; i += NTH) { sm.Tm[i] = M::cvt(0.f); sm.P[i] = M::cvt(0.f); }
  for (int i = tid; i < C * K::LDF; i += NTH) { sm.Mf[i] = 0.f; sm.Xf[i] = 0.f; }

  // State slabs of this wave, as accumulator tiles: Sacc[sl][ti] holds
  // S[16 ti + 4 g + e][col0 + c16], e = 0..3.
  f32x4 Sacc[K::SPW][K::NTK];
#pragma unroll
  for (int sl = 0; sl < K::SPW; ++sl) {
    const int slab = wave + NW * sl;
    const int col = vb * DVB + 16 * slab + c16;
#pragma unroll
    for (int ti = 0; ti < K::NTK; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Sacc[sl][ti][e] = (S0 != nullptr && slab < K::NSLAB)
                              ? S0[(bh * DK + 16 * ti + 4 * g + e) * DV + col]
                              : 0.f;
  }

  const int cg = tid % K::NCG, rg = tid / K::NCG;
  const bool pro = rg < K::NRG;
  const int ch0 = 8 * cg;
  const int nchunks = (T + C - 1) / C;

  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * C;
    const int valid = min(C, T - t0);
    __syncthreads();  // the previous chunk is done with every LDS tile

    // ---- value tiles for this wave's slabs (registers, accumulator layout)
    f32x4 R[K::SPW][K::NT];
#pragma unroll
    for (int sl = 0; sl < K::SPW; ++sl) {
      const int col = vb * DVB + 16 * (wave + NW * sl) + c16;
#pragma unroll
      for (int tr = 0; tr < K::NT; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tr + 4 * g + e;
          R[sl][tr][e] = (r < valid && wave + NW * sl < K::NSLAB) ? load_scalar(v, tok(t0 + r) * DV + col) : 0.f;
        }
    }

    // ---- 1. decay scan and operand tiles
    f32x8 lg[K::RPG];
    if (pro) {
      f32x8 run;
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] = 1.f;
#pragma unroll
      for (int rr = 0; rr < K::RPG; ++rr) {
        const int r = rg * K::RPG + rr;
        if (r < valid) {
          const f32x8 a = load8f(alpha + tok(t0 + r) * DK + ch0);
#pragma unroll
          for (int e = 0; e < 8; ++e) run[e] *= a[e];
        }
        lg[rr] = run;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.scan[rg * DK + ch0 + e] = run[e];
    }
    if (tid < C) sm.beta[tid] = (tid < valid) ? load_scalar(beta, tok(t0 + tid)) : 0.f;
    __syncthreads();
    if (tid < DK) {  // exclusive products of the row-group totals, per channel
      float p = 1.f;
      for (int gg = 0; gg < K::NRG; ++gg) {
        const float x = sm.scan[gg * DK + tid];
        sm.scan[gg * DK + tid] = p;
        p *= x;
      }
      sm.gC[tid] = p;
    }
    __syncthreads();
    if (pro) {
      f32x8 pre, gc;
#pragma unroll
      for (int e = 0; e < 8; ++e) { pre[e] = sm.scan[rg * DK + ch0 + e]; gc[e] = sm.gC[ch0 + e]; }
#pragma unroll
      for (int rr = 0; rr < K::RPG; ++rr) {
        const int r = rg * K::RPG + rr;
        f32x8 kk, qq;
        if (r < valid) {
          kk = load8f(k + tok(t0 + r) * DK + ch0);
          qq = load8f(q + tok(t0 + r) * DK + ch0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) kk[e] = qq[e] = 0.f;
        }
        f32x8 kp, qp, km;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gam = lg[rr][e] * pre[e];
          const float inv = __builtin_amdgcn_rcpf(gam);
          kp[e] = kk[e] * gam;
          qp[e] = qq[e] * gam;
          km[e] = kk[e] * inv;
        }
        M::store8(&sm.Kp[r * K::LDK + ch0], kp);
        M::store8(&sm.Qp[r * K::LDK + ch0], qp);
        M::store8(&sm.Km[r * K::LDK + ch0], km);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.KbT[(ch0 + e) * K::LDC + r] = M::cvt(km[e] * gc[e]);
      }
    }
    __syncthreads();

    // ---- 2. lower-triangular tiles of A (as Diag(beta) A, fp32) and P
    {
      constexpr int NPAIR = K::NT * (K::NT + 1) / 2;
      for (int job = wave; job < 2 * NPAIR; job += NW) {
        const bool isP = job & 1;
        int tr = 0, tc = job >> 1;
        while (tc > tr) { tc -= tr + 1; ++tr; }
        const lds_t* arow = (isP ? sm.Qp : sm.Kp) + (16 * tr + c16) * K::LDK;
        const lds_t* brow = sm.Km + (16 * tc + c16) * K::LDK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < K::NKS; ++s) {
          const int kb = 32 * s + 4 * g;
          if (K::KODD && s == K::NKS - 1)
            acc = M::mma(M::half(arow + kb), M::half(brow + kb), acc);
          else
            acc = M::mma(M::pair(arow + kb, arow + kb + 16), M::pair(brow + kb, brow + kb + 16), acc);
        }
        const int jc = 16 * tc + c16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tr + 4 * g + e;
          if (isP)
            sm.P[r * K::LDC + jc] = M::cvt(jc <= r ? acc[e] : 0.f);
          else
            sm.Mf[r * K::LDF + jc] = jc < r ? sm.beta[r] * acc[e] : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- 3. X = (I + Mf)^{-1}: diagonal 16x16 blocks by substitution
    for (int bi = wave; bi < K::NT; bi += NW) {
      if (lane < 16) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* mrow = &sm.Mf[(16 * bi + r) * K::LDF + 16 * bi];
          float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
          for (int j = 0; j < r; ++j) acc -= mrow[j] * x[j];
          x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Xf[(16 * bi + r) * K::LDF + 16 * bi + lane] = x[r];
      }
    }
    // off-diagonal blocks, one distance at a time:
    //   X_ab = -X_aa * sum_{c=b}^{a-1} Mf_ac X_cb
    for (int d = 1; d < K::NT; ++d) {
      __syncthreads();
      for (int bb = wave; bb < K::NT - d; bb += NW) {
        const int aa = bb + d;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int cc = bb; cc < aa; ++cc) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float av = sm.Mf[(16 * aa + c16) * K::LDF + 16 * cc + 4 * s + g];
            const float bv = sm.Xf[(16 * cc + 4 * s + g) * K::LDF + 16 * bb + c16];
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, y, 0, 0, 0);
          }
        }
        f32x4 xo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float av = sm.Xf[(16 * aa + c16) * K::LDF + 16 * aa + 4 * g + s];
          xo = __builtin_amdgcn_mfma_f32_16x16x4f32(av, y[s], xo, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Xf[(16 * aa + 4 * g + e) * K::LDF + 16 * bb + c16] = -xo[e];
      }
    }
    __syncthreads();
    // Tm = X Diag(beta), lower triangle
    for (int i = tid; i < C * C; i += NTH) {
      const int r = i / C, c = i % C;
      if (c <= r) sm.Tm[r * K::LDC + c] = M::cvt(sm.Xf[r * K::LDF + c] * sm.beta[c]);
    }
    __syncthreads();

    // ---- 4. per-slab state pass and output
#pragma unroll
    for (int sl = 0; sl < K::SPW; ++sl) {
      const int slab = wave + NW * sl;
      if (slab >= K::NSLAB) break;
      const int col = vb * DVB + 16 * slab + c16;
      f32x4* Sa = Sacc[sl];
      f32x4* Rv = R[sl];

      frag sfr[K::NKS];
#pragma unroll
      for (int s = 0; s < K::NKS; ++s) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        sfr[s] = M::from_acc(Sa[2 * s], (K::KODD && s == K::NKS - 1) ? z : Sa[2 * s + 1]);
      }
      // R = V - K+ S
#pragma unroll
      for (int tr = 0; tr < K::NT; ++tr) {
        const lds_t* arow = sm.Kp + (16 * tr + c16) * K::LDK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < K::NKS; ++s) {
          const int kb = 32 * s + 4 * g;
          const frag a = (K::KODD && s == K::NKS - 1) ? M::half(arow + kb) : M::pair(arow + kb, arow + kb + 16);
          acc = M::mma(a, sfr[s], acc);
        }
        Rv[tr] -= acc;
      }
      frag rfr[K::NCS];
#pragma unroll
      for (int s = 0; s < K::NCS; ++s) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        rfr[s] = M::from_acc(Rv[2 * s], (K::CODD && s == K::NCS - 1) ? z : Rv[2 * s + 1]);
      }
      // U = Tm R  (Tm lower triangular: k-steps up to the diagonal tile)
      f32x4 U[K::NT];
#pragma unroll
      for (int tr = 0; tr < K::NT; ++tr) {
        const lds_t* arow = sm.Tm + (16 * tr + c16) * K::LDC;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s <= tr / 2; ++s) {
          const int kb = 32 * s + 4 * g;
          const frag a = (K::CODD && s == K::NCS - 1) ? M::half(arow + kb) : M::pair(arow + kb, arow + kb + 16);
          acc = M::mma(a, rfr[s], acc);
        }
        U[tr] = acc;
      }
      frag ufr[K::NCS];
#pragma unroll
      for (int s = 0; s < K::NCS; ++s) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        ufr[s] = M::from_acc(U[2 * s], (K::CODD && s == K::NCS - 1) ? z : U[2 * s + 1]);
      }
      // O = Q+ S + P U
#pragma unroll
      for (int tr = 0; tr < K::NT; ++tr) {
        const lds_t* qrow = sm.Qp + (16 * tr + c16) * K::LDK;
        const lds_t* prow = sm.P + (16 * tr + c16) * K::LDC;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < K::NKS; ++s) {
          const int kb = 32 * s + 4 * g;
          const frag a = (K::KODD && s == K::NKS - 1) ? M::half(qrow + kb) : M::pair(qrow + kb, qrow + kb + 16);
          acc = M::mma(a, sfr[s], acc);
        }
#pragma unroll
        for (int s = 0; s <= tr / 2; ++s) {
          const int kb = 32 * s + 4 * g;
          const frag a = (K::CODD && s == K::NCS - 1) ? M::half(prow + kb) : M::pair(prow + kb, prow + kb + 16);
          acc = M::mma(a, ufr[s], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tr + 4 * g + e;
          if (r < valid) store_scalar(o, tok(t0 + r) * DV + col, acc[e]);
        }
      }
      // S <- Diag(gamma_C) S + Kbar^T U
#pragma unroll
      for (int ti = 0; ti < K::NTK; ++ti) {
        const lds_t* arow = sm.KbT + (16 * ti + c16) * K::LDC;
        f32x4 acc = Sa[ti];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= sm.gC[16 * ti + 4 * g + e];
#pragma unroll
        for (int s = 0; s < K::NCS; ++s) {
          const int kb = 32 * s + 4 * g;
          const frag a = (K::CODD && s == K::NCS - 1) ? M::half(arow + kb) : M::pair(arow + kb, arow + kb + 16);
          acc = M::mma(a, ufr[s], acc);
        }
        Sa[ti] = acc;
      }
    }
  }

  if (ST != nullptr) {
#pragma unroll
    for (int sl = 0; sl < K::SPW; ++sl) {
      const int slab = wave + NW * sl;
      if (slab >= K::NSLAB) break;
      const int col = vb * DVB + 16 * slab + c16;
#pragma unroll
      for (int ti = 0; ti < K::NTK; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e) ST[(bh * DK + 16 * ti + 4 * g + e) * DV + col] = Sacc[sl][ti][e];
    }
  }
}

template <typename E, int DK, int DVB, int C>
hipError_t launch_t(const PrefillArgs& a) {
  using St = typename E::storage;
  dim3 grid(a.d_v / DVB, a.H, a.B);
  hipLaunchKernelGGL((prefill_kernel<E, DK, DVB, C>), grid, dim3(NTH), 0, a.stream,
                     static_cast<const St*>(a.q), static_cast<const St*>(a.k),
                     static_cast<const St*>(a.v), static_cast<const St*>(a.alpha),
                     static_cast<const St*>(a.beta), a.S0, static_cast<St*>(a.o), a.S_T, a.T, a.H,
                     a.d_v);
  return hipGetLastError();
}

template <typename E, int DK, int DVB, int C>
constexpr bool fits() { return Cfg<E, DK, DVB, C>::smem_bytes <= 160 * 1024; }

// Value-block width: 64 columns (4 waves x one 16-column slab), or all of
// d_v when it is narrower.
constexpr int dvb_for(int dv) { return dv < 64 ? dv : 64; }

template <typename E, int DK, int C>
hipError_t dispatch_dv(const PrefillArgs& a, bool dry) {
  switch (a.d_v) {
#define KDA_CASE(DV)                                                             \
  case DV:                                                                       \
    if constexpr (fits<E, DK, dvb_for(DV), C>()) {                               \
      return dry ? hipSuccess : launch_t<E, DK, dvb_for(DV), C>(a);              \
    } else {                                                                     \
      return hipErrorNotSupported;                                               \
    }
    KDA_CASE(16)
    KDA_CASE(32)
    KDA_CASE(64)
    KDA_CASE(128)
#undef KDA_CASE
  }
  return hipErrorNotSupported;
}

template <typename E, int DK>
hipError_t dispatch_c(const PrefillArgs& a, bool dry) {
  switch (a.chunk) {
    case 16: return dispatch_dv<E, DK, 16>(a, dry);
    case 32: return dispatch_dv<E, DK, 32>(a, dry);
    case 64: return dispatch_dv<E, DK, 64>(a, dry);
  }
  return hipErrorNotSupported;
}

template <typename E>
hipError_t dispatch_dk(const PrefillArgs& a, bool dry) {
  switch (a.d_k) {
    case 16: return dispatch_c<E, 16>(a, dry);
    case 32: return dispatch_c<E, 32>(a, dry);
    case 64: return dispatch_c<E, 64>(a, dry);
    case 128: return dispatch_c<E, 128>(a, dry);
  }
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
  return a.bf16 ? dispatch_dk<Bf16>(a, false) : dispatch_dk<F32>(a, false);
}

bool prefill_supported(bool bf16, int d_k, int d_v, int chunk) {
  PrefillArgs a{};
  a.d_k = d_k; a.d_v = d_v; a.chunk = chunk; a.bf16 = bf16;
  return (bf16 ? dispatch_dk<Bf16>(a, true) : dispatch_dk<F32>(a, true)) == hipSuccess;
}

}  // namespace kda
