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
// Two kernels.
//   chunk_prep_kernel: everything that does not depend on S, for every
//     chunk of every (batch, head) at once (no sequential dependency).  Per
//     chunk it scans the cumulative decay, forms K+, K-, Q+, Kbar, runs the
//     Gram products on the matrix cores, inverts the unit lower-triangular
//     system in fp32, and writes five operand tiles (K+, Q+, Kbar^T, Tm, P)
//     plus gamma_C into a workspace slot, already in the per-lane order the
//     MFMA operands need.  Each workgroup walks a strided list of chunks and
//     prefetches the next chunk's inputs into registers while it works.
//   state_pass_kernel: one workgroup per (batch, head, value block), one
//     wave per 16-column slab of the fp32 state, which lives in accumulator
//     registers for the whole sequence.  It walks the chunks in order; the
//     next chunk's workspace slot streams into the other half of a
//     double-buffered LDS area (direct global->LDS loads) while the current
//     chunk's five products run.
//
// MFMA operand convention.  A 16x16 tile product over a k range of 32 takes
// 8 values per lane; lane (g = lane/16, c = lane%16) holds row/column c and
// k indices {32s+4g+e, 32s+16+4g+e : e = 0..3}.  That is exactly what a lane
// holds of two vertically stacked accumulator tiles, so accumulators become
// operands without data movement; the workspace stores every operand tile
// in this order, one 16-byte (bf16) or 32-byte (fp32) fragment per lane.
// The reduction does not depend on which k each (lane, element) slot
// carries as long as both operands agree.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// ----------------------------------------------------------------- helpers
template <typename St>
struct Raw8;  // 8 consecutive token-tensor elements as loaded from memory
template <>
struct Raw8<uint16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const uint16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ f32x8 unpack() const {
    f32x8 x;
    x[0] = __uint_as_float(r.x << 16); x[1] = __uint_as_float(r.x & 0xffff0000u);
    x[2] = __uint_as_float(r.y << 16); x[3] = __uint_as_float(r.y & 0xffff0000u);
    x[4] = __uint_as_float(r.z << 16); x[5] = __uint_as_float(r.z & 0xffff0000u);
    x[6] = __uint_as_float(r.w << 16); x[7] = __uint_as_float(r.w & 0xffff0000u);
    return x;
  }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ f32x8 unpack() const { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
};

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
  static __device__ __forceinline__ frag from8(f32x8 x) {
    frag r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    return r;
  }
  static __device__ __forceinline__ void store8(lds_t* p, f32x8 x) { *reinterpret_cast<frag*>(p) = from8(x); }
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
  static __device__ __forceinline__ frag from8(f32x8 x) { return x; }
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

// Shapes shared by both kernels.
template <typename E, int DK, int C>
struct Shape {
  using M = Mma<E>;
  using lds_t = typename M::lds_t;
  using frag = typename M::frag;
  static constexpr int NT = C / 16;          // 16-row tiles per chunk
  static constexpr int NTK = DK / 16;        // 16-row tiles of the state
  static constexpr int NKS = (NTK + 1) / 2;  // 32-wide k-steps over d_k
  static constexpr bool KODD = (NTK & 1) != 0;
  static constexpr int NCS = (NT + 1) / 2;   // 32-wide k-steps over the chunk
  static constexpr bool CODD = (NT & 1) != 0;
  // Workspace slot: operand tiles as [tile][k-step][lane] fragments.
  static constexpr int FB = 8 * static_cast<int>(sizeof(lds_t));  // bytes per lane fragment
  static constexpr int FRAG = 64 * FB;                              // bytes per wave fragment
  static constexpr int OFF_KP = 0;
  static constexpr int OFF_QP = OFF_KP + NT * NKS * FRAG;
  static constexpr int OFF_KB = OFF_QP + NT * NKS * FRAG;
  static constexpr int OFF_TM = OFF_KB + NTK * NCS * FRAG;
  static constexpr int OFF_PP = OFF_TM + NT * NCS * FRAG;
  static constexpr int OFF_GC = OFF_PP + NT * NCS * FRAG;
  static constexpr int SLOT = ((OFF_GC + DK * 4) + 1023) / 1024 * 1024;  // whole 1 KiB copy units
};

// ======================================================== chunk preparation
constexpr int NTH_PREP = 256;
constexpr int NW_PREP = NTH_PREP / 64;

template <typename E, int DK, int C>
struct PrepCfg {
  using S = Shape<E, DK, C>;
  using lds_t = typename S::lds_t;
  static constexpr int NCG = DK / 8;  // 8-channel groups
  static constexpr int NRG0 = NTH_PREP / NCG;
  static constexpr int NRG = NRG0 < C ? NRG0 : C;  // row groups in use
  static constexpr int RPG = C / NRG;               // rows per row group
  static constexpr int LDK = DK + S::M::PAD;
  static constexpr int LDC = C + S::M::PAD;
  static constexpr int LDF = C + 4;  // fp32 C x C tiles (16-byte aligned rows)
  static_assert(NRG * RPG == C && NCG * NRG <= NTH_PREP, "prologue map");
  struct Smem {
    alignas(16) lds_t Kp[C * LDK];
    alignas(16) lds_t Km[C * LDK];
    alignas(16) lds_t Qp[C * LDK];
    alignas(16) lds_t KbT[DK * LDC];
    alignas(16) float Mf[C * LDF];  // Diag(beta) A, strictly lower
    alignas(16) float Xf[C * LDF];  // (I + Diag(beta) A)^{-1}, lower
    alignas(16) float gC[DK];
    alignas(16) float beta[C];
    alignas(16) float scan[NRG * DK];
  };
};

template <typename E, int DK, int C>
__global__ __launch_bounds__(NTH_PREP) void chunk_prep_kernel(
    const typename E::storage* __restrict__ q, const typename E::storage* __restrict__ k,
    const typename E::storage* __restrict__ alpha, const typename E::storage* __restrict__ beta,
    char* __restrict__ ws, int T, int H, int nchunk, int ntask) {
  using S = Shape<E, DK, C>;
  using P = PrepCfg<E, DK, C>;
  using M = typename S::M;
  using lds_t = typename S::lds_t;
  using frag = typename S::frag;
  using St = typename E::storage;
  __shared__ typename P::Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int cg = tid % P::NCG, rg = tid / P::NCG;
  const bool pro = rg < P::NRG;
  const int ch0 = 8 * cg;

  // Upper parts of Mf and Xf are never written per chunk: zero them once.
  for (int i = tid; i < C * P::LDF; i += NTH_PREP) { sm.Mf[i] = 0.f; sm.Xf[i] = 0.f; }

  // Token row of (task, r), clamped into the sequence so loads stay in bounds.
  auto rowptr = [&](int task, int r) -> long {
    const int chain = task / nchunk, n = task - chain * nchunk;
    const int b = chain / H, h = chain - b * H;
    const int t = min(n * C + r, T - 1);
    return (static_cast<long>(b) * T + t) * H + h;
  };

  Raw8<St> ra[P::RPG], rk[P::RPG], rq[P::RPG];
  auto prefetch = [&](int task) {
    if (task < ntask && pro) {
#pragma unroll
      for (int rr = 0; rr < P::RPG; ++rr) {
        const long row = rowptr(task, rg * P::RPG + rr);
        ra[rr].load(alpha + row * DK + ch0);
        rk[rr].load(k + row * DK + ch0);
        rq[rr].load(q + row * DK + ch0);
      }
    }
  };
  prefetch(blockIdx.x);

  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int n = task % nchunk;
    const int valid = min(C, T - n * C);
    char* slot = ws + static_cast<long>(task) * S::SLOT;

    // ---- 1. decay scan, from the prefetched registers
    f32x8 lg[P::RPG], kk[P::RPG], qq[P::RPG];
    __syncthreads();  // the previous task is done with every LDS tile
    if (pro) {
      f32x8 run;
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] = 1.f;
#pragma unroll
      for (int rr = 0; rr < P::RPG; ++rr) {
        const bool ok = rg * P::RPG + rr < valid;
        const f32x8 a = ra[rr].unpack();
        kk[rr] = rk[rr].unpack();
        qq[rr] = rq[rr].unpack();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          run[e] *= ok ? a[e] : 1.f;
          kk[rr][e] = ok ? kk[rr][e] : 0.f;
          qq[rr][e] = ok ? qq[rr][e] : 0.f;
        }
        lg[rr] = run;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.scan[rg * DK + ch0 + e] = run[e];
    }
    if (tid < C) {
      const float bv = load_scalar(beta, rowptr(task, tid));
      sm.beta[tid] = tid < valid ? bv : 0.f;
    }
    prefetch(task + gridDim.x);  // next task's inputs load while this one computes
    __syncthreads();
    if (tid < DK) {  // exclusive products of the row-group totals, per channel
      float tot[P::NRG];
#pragma unroll
      for (int gg = 0; gg < P::NRG; ++gg) tot[gg] = sm.scan[gg * DK + tid];
      float p = 1.f;
#pragma unroll
      for (int gg = 0; gg < P::NRG; ++gg) {
        sm.scan[gg * DK + tid] = p;
        p *= tot[gg];
      }
      sm.gC[tid] = p;
    }
    __syncthreads();

    // ---- 2. decay-scaled operand tiles
    if (pro) {
      f32x8 pre, gc;
#pragma unroll
      for (int e = 0; e < 8; ++e) { pre[e] = sm.scan[rg * DK + ch0 + e]; gc[e] = sm.gC[ch0 + e]; }
#pragma unroll
      for (int rr = 0; rr < P::RPG; ++rr) {
        const int r = rg * P::RPG + rr;
        f32x8 kp, qp, km;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gam = lg[rr][e] * pre[e];
          const float inv = __builtin_amdgcn_rcpf(gam);
          kp[e] = kk[rr][e] * gam;
          qp[e] = qq[rr][e] * gam;
          km[e] = kk[rr][e] * inv;
        }
        M::store8(&sm.Kp[r * P::LDK + ch0], kp);
        M::store8(&sm.Qp[r * P::LDK + ch0], qp);
        M::store8(&sm.Km[r * P::LDK + ch0], km);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.KbT[(ch0 + e) * P::LDC + r] = M::cvt(km[e] * gc[e]);
      }
    }
    __syncthreads();

    // ---- 3. Gram tiles, P fragments, and the K+ / Q+ / Kbar^T fragments
    {
      // A tile (tr, tc), tc <= tr: A[16tr+4g+e][16tc+c16] -> Diag(beta) A, fp32 LDS.
      constexpr int NPAIR = S::NT * (S::NT + 1) / 2;
      int job = 0;
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int tc = 0; tc <= tr; ++tc, ++job) {
          if (job % NW_PREP != wave) continue;
          const lds_t* arow = sm.Kp + (16 * tr + c16) * P::LDK;
          const lds_t* brow = sm.Km + (16 * tc + c16) * P::LDK;
          frag af[S::NKS], bf[S::NKS];
#pragma unroll
          for (int s = 0; s < S::NKS; ++s) {
            const int kb = 32 * s + 4 * g;
            const bool h = S::KODD && s == S::NKS - 1;
            af[s] = h ? M::half(arow + kb) : M::pair(arow + kb, arow + kb + 16);
            bf[s] = h ? M::half(brow + kb) : M::pair(brow + kb, brow + kb + 16);
          }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < S::NKS; ++s) acc = M::mma(af[s], bf[s], acc);
          const int jc = 16 * tc + c16;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * tr + 4 * g + e;
            sm.Mf[r * P::LDF + jc] = jc < r ? sm.beta[r] * acc[e] : 0.f;
          }
        }
      // P fragments (tr, s), s <= tr/2, from P^T tiles: the accumulator of
      // the product K- Q+^T holds P[16tr+c16][16tc+4g+e] in lane (g, c16),
      // i.e. exactly the operand order.
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int s = 0; s <= tr / 2; ++s, ++job) {
          if (job % NW_PREP != wave) continue;
          const lds_t* brow = sm.Qp + (16 * tr + c16) * P::LDK;
          f32x4 half_acc[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int tc = 2 * s + hh;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (tc <= tr) {
              const lds_t* arow = sm.Km + (16 * tc + c16) * P::LDK;
              frag af[S::NKS], bf[S::NKS];
#pragma unroll
              for (int ks = 0; ks < S::NKS; ++ks) {
                const int kb = 32 * ks + 4 * g;
                const bool h = S::KODD && ks == S::NKS - 1;
                af[ks] = h ? M::half(arow + kb) : M::pair(arow + kb, arow + kb + 16);
                bf[ks] = h ? M::half(brow + kb) : M::pair(brow + kb, brow + kb + 16);
              }
#pragma unroll
              for (int ks = 0; ks < S::NKS; ++ks) acc = M::mma(af[ks], bf[ks], acc);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (16 * tc + 4 * g + e > 16 * tr + c16) acc[e] = 0.f;
            }
            half_acc[hh] = acc;
          }
          frag* dst = reinterpret_cast<frag*>(slot + S::OFF_PP + (tr * S::NCS + s) * S::FRAG);
          dst[lane] = M::from_acc(half_acc[0], half_acc[1]);
        }
      // K+, Q+ fragments (rows r, k = channels) and Kbar^T fragments (rows =
      // channels, k = r) copied from LDS into the workspace.
#pragma unroll
      for (int t = 0; t < S::NT; ++t)
#pragma unroll
        for (int s = 0; s < S::NKS; ++s)
#pragma unroll
          for (int w2 = 0; w2 < 2; ++w2, ++job) {
            if (job % NW_PREP != wave) continue;
            const lds_t* row = (w2 ? sm.Qp : sm.Kp) + (16 * t + c16) * P::LDK;
            const int kb = 32 * s + 4 * g;
            const frag f = (S::KODD && s == S::NKS - 1) ? M::half(row + kb) : M::pair(row + kb, row + kb + 16);
            frag* dst = reinterpret_cast<frag*>(slot + (w2 ? S::OFF_QP : S::OFF_KP) + (t * S::NKS + s) * S::FRAG);
            dst[lane] = f;
          }
#pragma unroll
      for (int t = 0; t < S::NTK; ++t)
#pragma unroll
        for (int s = 0; s < S::NCS; ++s, ++job) {
          if (job % NW_PREP != wave) continue;
          const lds_t* row = sm.KbT + (16 * t + c16) * P::LDC;
          const int kb = 32 * s + 4 * g;
          const frag f = (S::CODD && s == S::NCS - 1) ? M::half(row + kb) : M::pair(row + kb, row + kb + 16);
          frag* dst = reinterpret_cast<frag*>(slot + S::OFF_KB + (t * S::NCS + s) * S::FRAG);
          dst[lane] = f;
        }
      (void)NPAIR;
      if (tid < DK) reinterpret_cast<float*>(slot + S::OFF_GC)[tid] = sm.gC[tid];
    }
    __syncthreads();

    // ---- 4. X = (I + Mf)^{-1}: diagonal 16x16 blocks by substitution
    for (int bi = wave; bi < S::NT; bi += NW_PREP) {
      if (lane < 16) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* mrow = &sm.Mf[(16 * bi + r) * P::LDF + 16 * bi];
          float m[16];
#pragma unroll
          for (int j = 0; j < r; ++j) m[j] = mrow[j];
          float a0 = (r == lane) ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
          for (int j = 0; j < r; j += 2) {
            a0 -= m[j] * x[j];
            if (j + 1 < r) a1 -= m[j + 1] * x[j + 1];
          }
          x[r] = a0 + a1;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Xf[(16 * bi + r) * P::LDF + 16 * bi + lane] = x[r];
      }
    }
    // off-diagonal blocks, one distance at a time:
    //   X_ab = -X_aa * sum_{c=b}^{a-1} Mf_ac X_cb
#pragma unroll
    for (int d = 1; d < S::NT; ++d) {
      __syncthreads();
      for (int bb = wave; bb < S::NT - d; bb += NW_PREP) {
        const int aa = bb + d;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int cc = bb; cc < aa; ++cc) {
          float av[4], bv[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            av[s] = sm.Mf[(16 * aa + c16) * P::LDF + 16 * cc + 4 * s + g];
            bv[s] = sm.Xf[(16 * cc + 4 * s + g) * P::LDF + 16 * bb + c16];
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) y = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], y, 0, 0, 0);
        }
        float av[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) av[s] = sm.Xf[(16 * aa + c16) * P::LDF + 16 * aa + 4 * g + s];
        f32x4 xo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) xo = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], y[s], xo, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Xf[(16 * aa + 4 * g + e) * P::LDF + 16 * bb + c16] = -xo[e];
      }
    }
    __syncthreads();

    // ---- 5. Tm = X Diag(beta) fragments (rows r, k = columns), s <= tr/2
    {
      int job = 0;
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int s = 0; s <= tr / 2; ++s, ++job) {
          if (job % NW_PREP != wave) continue;
          const float* xrow = sm.Xf + (16 * tr + c16) * P::LDF;
          const int kb = 32 * s + 4 * g;
          f32x8 t8;
          const f32x4 lo = *reinterpret_cast<const f32x4*>(xrow + kb);
#pragma unroll
          for (int e = 0; e < 4; ++e) t8[e] = lo[e] * sm.beta[kb + e];
          if (S::CODD && s == S::NCS - 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) t8[4 + e] = 0.f;
          } else {
            const f32x4 hi = *reinterpret_cast<const f32x4*>(xrow + kb + 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) t8[4 + e] = hi[e] * sm.beta[kb + 16 + e];
          }
          frag* dst = reinterpret_cast<frag*>(slot + S::OFF_TM + (tr * S::NCS + s) * S::FRAG);
          dst[lane] = M::from8(t8);
        }
    }
  }
}

// ============================================================ state pass
constexpr size_t kLdsLimit = 160 * 1024;

template <typename E, int DK, int DVB, int C>
struct PassCfg {
  using S = Shape<E, DK, C>;
  static constexpr int NWB = DVB / 16;  // one wave per 16-column slab
  static constexpr int NTH = 64 * NWB;
  static constexpr int SLOT = S::SLOT;
  // Double-buffer the slot when two fit in LDS, else stream it after compute.
  static constexpr int NBUF = 2 * static_cast<size_t>(SLOT) <= kLdsLimit ? 2 : 1;
  static constexpr size_t smem_bytes = NBUF * static_cast<size_t>(SLOT);
};

template <typename E, int DK, int DVB, int C>
__global__ __launch_bounds__((PassCfg<E, DK, DVB, C>::NTH)) void state_pass_kernel(
    const char* __restrict__ ws, const typename E::storage* __restrict__ v,
    const float* __restrict__ S0, typename E::storage* __restrict__ o, float* __restrict__ ST,
    int T, int H, int DV, int nchunk) {
  using S = Shape<E, DK, C>;
  using K = PassCfg<E, DK, DVB, C>;
  using M = typename S::M;
  using frag = typename S::frag;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int chain = blockIdx.x, vb = blockIdx.y;
  const int b = chain / H, h = chain - b * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int col = vb * DVB + 16 * wave + c16;
  const long bh = chain;
  auto tok = [&](int t) -> long { return (static_cast<long>(b) * T + t) * H + h; };
  const char* wsb = ws + static_cast<long>(chain) * nchunk * K::SLOT;

  // Copy one workspace slot into LDS half `buf`, 1 KiB per wave instruction.
  auto stage = [&](int n, int buf) {
    const char* src = wsb + static_cast<long>(n) * K::SLOT;
    char* dst = lds + buf * K::SLOT;
    for (int u = wave; u < K::SLOT / 1024; u += K::NWB)
      __builtin_amdgcn_global_load_lds((gvoid_t*)(src + u * 1024 + lane * 16), (lvoid_t*)(dst + u * 1024), 16, 0, 0);
  };
  auto load_v = [&](int n, f32x4* R) {
#pragma unroll
    for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = n * C + 16 * tr + 4 * g + e;
        const float x = load_scalar(v, tok(min(t, T - 1)) * DV + col);
        R[tr][e] = t < T ? x : 0.f;
      }
  };

  // State slab as accumulator tiles: Sa[ti] holds S[16 ti + 4 g + e][col].
  f32x4 Sa[S::NTK];
#pragma unroll
  for (int ti = 0; ti < S::NTK; ++ti)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Sa[ti][e] = S0 != nullptr ? S0[(bh * DK + 16 * ti + 4 * g + e) * DV + col] : 0.f;

  f32x4 Rn[S::NT];
  if (nchunk > 0) {
    stage(0, 0);
    load_v(0, Rn);
  }
  for (int n = 0; n < nchunk; ++n) {
    f32x4 R[S::NT];
#pragma unroll
    for (int tr = 0; tr < S::NT; ++tr) R[tr] = Rn[tr];
    __builtin_amdgcn_s_waitcnt(0);  // this chunk's slot has landed in LDS
    __syncthreads();                // ... for every wave; the other half is free
    if (n + 1 < nchunk) {
      if (K::NBUF == 2) stage(n + 1, (n + 1) & 1);
      load_v(n + 1, Rn);
    }
    const char* sl = lds + (K::NBUF == 2 ? (n & 1) : 0) * K::SLOT;
    auto fr = [&](int off, int idx) -> frag {
      return reinterpret_cast<const frag*>(sl + off + idx * S::FRAG)[lane];
    };
    const float* gC = reinterpret_cast<const float*>(sl + S::OFF_GC);
    const int t0 = n * C;

    frag sfr[S::NKS];
#pragma unroll
    for (int s = 0; s < S::NKS; ++s) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      sfr[s] = M::from_acc(Sa[2 * s], (S::KODD && s == S::NKS - 1) ? z : Sa[2 * s + 1]);
    }
    // R = V - K+ S
#pragma unroll
    for (int tr = 0; tr < S::NT; ++tr) {
      frag a[S::NKS];
#pragma unroll
      for (int s = 0; s < S::NKS; ++s) a[s] = fr(S::OFF_KP, tr * S::NKS + s);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S::NKS; ++s) acc = M::mma(a[s], sfr[s], acc);
      R[tr] -= acc;
    }
    frag rfr[S::NCS];
#pragma unroll
    for (int s = 0; s < S::NCS; ++s) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      rfr[s] = M::from_acc(R[2 * s], (S::CODD && s == S::NCS - 1) ? z : R[2 * s + 1]);
    }
    // U = Tm R  (Tm lower triangular: k-steps up to the diagonal tile)
    f32x4 U[S::NT];
#pragma unroll
    for (int tr = 0; tr < S::NT; ++tr) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= tr / 2; ++s) acc = M::mma(fr(S::OFF_TM, tr * S::NCS + s), rfr[s], acc);
      U[tr] = acc;
    }
    frag ufr[S::NCS];
#pragma unroll
    for (int s = 0; s < S::NCS; ++s) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      ufr[s] = M::from_acc(U[2 * s], (S::CODD && s == S::NCS - 1) ? z : U[2 * s + 1]);
    }
    // O = Q+ S + P U
#pragma unroll
    for (int tr = 0; tr < S::NT; ++tr) {
      frag a[S::NKS];
#pragma unroll
      for (int s = 0; s < S::NKS; ++s) a[s] = fr(S::OFF_QP, tr * S::NKS + s);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S::NKS; ++s) acc = M::mma(a[s], sfr[s], acc);
#pragma unroll
      for (int s = 0; s <= tr / 2; ++s) acc = M::mma(fr(S::OFF_PP, tr * S::NCS + s), ufr[s], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * tr + 4 * g + e;
        if (t < T) store_scalar(o, tok(t) * DV + col, acc[e]);
      }
    }
    // S <- Diag(gamma_C) S + Kbar^T U
#pragma unroll
    for (int ti = 0; ti < S::NTK; ++ti) {
      frag a[S::NCS];
#pragma unroll
      for (int s = 0; s < S::NCS; ++s) a[s] = fr(S::OFF_KB, ti * S::NCS + s);
      f32x4 acc = Sa[ti];
      const f32x4 gc = *reinterpret_cast<const f32x4*>(gC + 16 * ti + 4 * g);
      acc *= gc;
#pragma unroll
      for (int s = 0; s < S::NCS; ++s) acc = M::mma(a[s], ufr[s], acc);
      Sa[ti] = acc;
    }
    if (K::NBUF == 1 && n + 1 < nchunk) {
      __syncthreads();  // every wave is done with the single slot
      stage(n + 1, 0);
    }
  }

  if (ST != nullptr) {
#pragma unroll
    for (int ti = 0; ti < S::NTK; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) ST[(bh * DK + 16 * ti + 4 * g + e) * DV + col] = Sa[ti][e];
  }
}

// ================================================================== host

// Value-block width of a state-pass workgroup: two 16-column slabs (one wave
// each), or all of d_v when it is 16.
constexpr int dvb_for(int dv) { return dv < 32 ? dv : 32; }

template <typename E, int DK, int C>
constexpr bool fits() {
  return sizeof(typename PrepCfg<E, DK, C>::Smem) <= kLdsLimit &&
         static_cast<size_t>(Shape<E, DK, C>::SLOT) <= kLdsLimit;
}

template <typename E, int DK, int C>
size_t slot_bytes() { return Shape<E, DK, C>::SLOT; }

int g_num_cus = 0;
int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

template <typename E, int DK, int C>
hipError_t launch_t(const PrefillArgs& a) {
  using St = typename E::storage;
  using S = Shape<E, DK, C>;
  const int nchunk = (a.T + C - 1) / C;
  const long ntask = static_cast<long>(a.B) * a.H * nchunk;
  char* ws = static_cast<char*>(a.workspace);
  if (ntask > 0) {
    const int grid = static_cast<int>(ntask < num_cus() ? ntask : num_cus());
    hipLaunchKernelGGL((chunk_prep_kernel<E, DK, C>), dim3(grid), dim3(NTH_PREP), 0, a.stream,
                       static_cast<const St*>(a.q), static_cast<const St*>(a.k),
                       static_cast<const St*>(a.alpha), static_cast<const St*>(a.beta), ws, a.T,
                       a.H, nchunk, static_cast<int>(ntask));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto pass = [&](auto dvb_tag) -> hipError_t {
    constexpr int DVB = decltype(dvb_tag)::value;
    using K = PassCfg<E, DK, DVB, C>;
    static bool attr_set = false;  // one-time opt-in to more than 64 KiB of LDS
    if (!attr_set) {
      const void* fn = reinterpret_cast<const void*>(&state_pass_kernel<E, DK, DVB, C>);
      hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(K::smem_bytes));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    hipLaunchKernelGGL((state_pass_kernel<E, DK, DVB, C>), dim3(a.B * a.H, a.d_v / DVB),
                       dim3(K::NTH), K::smem_bytes, a.stream, ws, static_cast<const St*>(a.v),
                       a.S0, static_cast<St*>(a.o), a.S_T, a.T, a.H, a.d_v, nchunk);
    return hipGetLastError();
  };
  (void)sizeof(S);
  if (a.d_v == 16) return pass(std::integral_constant<int, 16>{});
  return pass(std::integral_constant<int, 32>{});
}

template <typename E, int DK>
hipError_t dispatch_c(const PrefillArgs& a, size_t* slot) {
  switch (a.chunk) {
#define KDA_CASE(CC)                                                      \
  case CC:                                                                \
    if constexpr (fits<E, DK, CC>()) {                                    \
      if (slot) { *slot = slot_bytes<E, DK, CC>(); return hipSuccess; }   \
      return launch_t<E, DK, CC>(a);                                      \
    } else {                                                              \
      return hipErrorNotSupported;                                        \
    }
    KDA_CASE(16)
    KDA_CASE(32)
    KDA_CASE(64)
#undef KDA_CASE
  }
  return hipErrorNotSupported;
}

template <typename E>
hipError_t dispatch_dk(const PrefillArgs& a, size_t* slot) {
  switch (a.d_k) {
    case 16: return dispatch_c<E, 16>(a, slot);
    case 32: return dispatch_c<E, 32>(a, slot);
    case 64: return dispatch_c<E, 64>(a, slot);
    case 128: return dispatch_c<E, 128>(a, slot);
  }
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
  return a.bf16 ? dispatch_dk<Bf16>(a, nullptr) : dispatch_dk<F32>(a, nullptr);
}

bool prefill_supported(bool bf16, int d_k, int d_v, int chunk) {
  size_t s = 0;
  return prefill_slot_bytes(bf16, d_k, d_v, chunk, &s);
}

bool prefill_slot_bytes(bool bf16, int d_k, int d_v, int chunk, size_t* slot) {
  PrefillArgs a{};
  a.d_k = d_k; a.d_v = d_v; a.chunk = chunk; a.bf16 = bf16;
  if (d_v != 16 && d_v != 32 && d_v != 64 && d_v != 128) return false;
  return (bf16 ? dispatch_dk<Bf16>(a, slot) : dispatch_dk<F32>(a, slot)) == hipSuccess;
}

}  // namespace kda
