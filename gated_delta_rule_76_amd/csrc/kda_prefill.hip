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
// Fused prologue (optional): from raw projections the prep kernel forms
// q / |q|, k / |k| per token and head, alpha = exp(-c softplus(g)) and
// beta = sigmoid(b) in fp32 before anything else; the state pass only reads
// the slot and v, so it is unaffected.
//
// Variants: a per-head scalar gate (Gated DeltaNet) is the same algebra with
// alpha broadcast over the channels; no gate sets alpha = 1.  Without the
// correction (additive linear memory, section 2.1) there is no erase term:
// A = 0, so Tm = Diag(beta) and R = V.
//
// Two kernels.
//   chunk_prep_kernel: everything that does not depend on S, for every
//     chunk of every (batch, head) at once (no sequential dependency).  Per
//     chunk it scans the cumulative decay, forms K+, K-, Q+, Kbar, runs the
//     Gram products on the matrix cores, inverts the unit lower-triangular
//     system in fp32, and writes five operand tiles (K+, Q+, Kbar^T, Tm, P)
//     plus gamma_C into a workspace slot, already in the per-lane order the
//     MFMA operands need (streaming stores: nothing re-reads them from L2
//     soon).  Each workgroup walks a strided list of chunks and prefetches
//     the next chunk's inputs into registers while it works.
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
//
// Bounds checks.  Every global index and run-time LDS destination below goes
// through chk() / chk_ok() (kda_check.h): in the checked build a wrong index
// is caught before the access; in the normal build they compile away.
#include <atomic>
#include <mutex>
#include <type_traits>
#include <utility>

#include "kda_check.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __attribute__((address_space(1))) void gvoid_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lvoid_t;

// Check sites of this unit (bits of the checked build's failure mask).
enum : int {
  kSiteQK = 0,         // prep: q and k rows
  kSiteAlpha = 1,      // prep: gate rows
  kSiteBeta = 2,       // prep: beta
  kSiteSlotStore = 3,  // prep: workspace slot stores
  kSiteSlotLoad = 4,   // pass: slot copies into LDS
  kSiteValue = 5,      // pass: value rows (copies and prefetch)
  kSiteOut = 6,        // pass: output rows
  kSiteS0 = 7,         // pass: initial state
  kSiteST = 8,         // pass: final state
  kSiteLds = 9,        // pass: LDS destinations of the direct loads
  kSitePrefetch = 10,  // pass: slot prefetch
  kSiteProbe = 11,     // the checked build's self-test
};

// ----------------------------------------------------------------- helpers
// Batched LDS reads for the state chain: 16-byte reads at addr + offsets
// issued back to back, then a single wait for all of them.  One asm
// statement each, so that the compiler neither places a wait between the
// reads nor moves them next to their uses (which serialises one LDS round
// trip per matrix product).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}
// 16 reads at addr + O + i * D, i = 0..15
template <int O, int D>
__device__ __forceinline__ void lds_read16(uint32_t a, u32x4 (&r)[16]) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:%17\n\tds_read_b128 %1, %16 offset:%18\n\t"
      "ds_read_b128 %2, %16 offset:%19\n\tds_read_b128 %3, %16 offset:%20\n\t"
      "ds_read_b128 %4, %16 offset:%21\n\tds_read_b128 %5, %16 offset:%22\n\t"
      "ds_read_b128 %6, %16 offset:%23\n\tds_read_b128 %7, %16 offset:%24\n\t"
      "ds_read_b128 %8, %16 offset:%25\n\tds_read_b128 %9, %16 offset:%26\n\t"
      "ds_read_b128 %10, %16 offset:%27\n\tds_read_b128 %11, %16 offset:%28\n\t"
      "ds_read_b128 %12, %16 offset:%29\n\tds_read_b128 %13, %16 offset:%30\n\t"
      "ds_read_b128 %14, %16 offset:%31\n\tds_read_b128 %15, %16 offset:%32\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
        "=&v"(r[14]), "=&v"(r[15])
      : "v"(a), "i"(O), "i"(O + D), "i"(O + 2 * D), "i"(O + 3 * D), "i"(O + 4 * D), "i"(O + 5 * D),
        "i"(O + 6 * D), "i"(O + 7 * D), "i"(O + 8 * D), "i"(O + 9 * D), "i"(O + 10 * D), "i"(O + 11 * D),
        "i"(O + 12 * D), "i"(O + 13 * D), "i"(O + 14 * D), "i"(O + 15 * D)
      : "memory");
}
// 6 reads at a + O + i * D and 8 reads at b + P + i * E
template <int O, int D, int P, int E>
__device__ __forceinline__ void lds_read6_8(uint32_t a, u32x4 (&r)[6], uint32_t b, u32x4 (&s)[8]) {
  asm volatile(
      "ds_read_b128 %0, %14 offset:%16\n\tds_read_b128 %1, %14 offset:%17\n\t"
      "ds_read_b128 %2, %14 offset:%18\n\tds_read_b128 %3, %14 offset:%19\n\t"
      "ds_read_b128 %4, %14 offset:%20\n\tds_read_b128 %5, %14 offset:%21\n\t"
      "ds_read_b128 %6, %15 offset:%22\n\tds_read_b128 %7, %15 offset:%23\n\t"
      "ds_read_b128 %8, %15 offset:%24\n\tds_read_b128 %9, %15 offset:%25\n\t"
      "ds_read_b128 %10, %15 offset:%26\n\tds_read_b128 %11, %15 offset:%27\n\t"
      "ds_read_b128 %12, %15 offset:%28\n\tds_read_b128 %13, %15 offset:%29\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(s[0]),
        "=&v"(s[1]), "=&v"(s[2]), "=&v"(s[3]), "=&v"(s[4]), "=&v"(s[5]), "=&v"(s[6]), "=&v"(s[7])
      : "v"(a), "v"(b), "i"(O), "i"(O + D), "i"(O + 2 * D), "i"(O + 3 * D), "i"(O + 4 * D),
        "i"(O + 5 * D), "i"(P), "i"(P + E), "i"(P + 2 * E), "i"(P + 3 * E), "i"(P + 4 * E),
        "i"(P + 5 * E), "i"(P + 6 * E), "i"(P + 7 * E)
      : "memory");
}

template <typename St>
struct Raw8;  // 8 consecutive token-tensor elements as loaded from memory
template <>
struct Raw8<uint16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const uint16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  // one value for all 8 slots: loaded here, broadcast by unpack_one (so the
  // load is not waited for until the value is used)
  __device__ __forceinline__ void load_one(const uint16_t* p) { r.x = *p; }
  __device__ __forceinline__ f32x8 unpack_one() const {
    const float x = __uint_as_float(r.x << 16);
    return f32x8{x, x, x, x, x, x, x, x};
  }
  __device__ __forceinline__ void ones() { r = uint4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}; }
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
  __device__ __forceinline__ void load_one(const float* p) { a.x = *p; }
  __device__ __forceinline__ f32x8 unpack_one() const {
    const float x = a.x;
    return f32x8{x, x, x, x, x, x, x, x};
  }
  __device__ __forceinline__ void ones() { a = b = f32x4{1.f, 1.f, 1.f, 1.f}; }
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
  static __device__ __forceinline__ void store4(lds_t* p, f32x4 x) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
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
  // Lower-triangular C x C operands keep only the fragments (tr, s) with
  // s <= tr / 2; tri(tr) = sum_{t < tr} (t / 2 + 1) is the index of (tr, 0)
  // in that list.
  static constexpr __host__ __device__ int tri(int tr) { return tr + ((tr - 1) * (tr - 1)) / 4; }
  static_assert(tri(0) == 0 && tri(1) == 1 && tri(2) == 2 && tri(3) == 4 && tri(4) == 6, "tri");
  static constexpr int NTRI = tri(NT);
  // Workspace slot: operand tiles as [tile][k-step][lane] fragments.
  static constexpr int FB = 8 * static_cast<int>(sizeof(lds_t));  // bytes per lane fragment
  static constexpr int FRAG = 64 * FB;                              // bytes per wave fragment
  static constexpr int OFF_KP = 0;
  static constexpr int OFF_QP = OFF_KP + NT * NKS * FRAG;
  static constexpr int OFF_KB = OFF_QP + NT * NKS * FRAG;
  static constexpr int OFF_TM = OFF_KB + NTK * NCS * FRAG;
  static constexpr int OFF_PP = OFF_TM + NTRI * FRAG;
  static constexpr int OFF_GC = OFF_PP + NTRI * FRAG;
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
  // Operand-tile layout.  The bf16 tiles K+, K- and Q+ with d_k a multiple
  // of 32 are kept in 16-byte chunks in matrix-core operand order: chunk
  // 4s + g of row r holds channels 32s + 4g .. +3 and 32s + 16 + 4g .. +3,
  // the eight values lane group g of a 16x16x32 product takes at k-step s,
  // so every operand fragment is one 16-byte LDS read, and rows are padded
  // by two chunks.  LDS serves 16-byte reads to 16 lanes at a time over 64
  // banks (within a half wave, the lanes whose lane / 4 has an even, or an
  // odd, number of set bits) and 8-byte writes to 16 consecutive lanes over
  // 32 banks.  With this layout the fragment reads are free of bank
  // conflicts, and so are the two 8-byte stores of each thread's eight
  // channels when the threads holding channels 64 .. 127 store their upper
  // four first (measured on gfx950: the row-major tile with 16-byte padding
  // took 8 conflict cycles per pair read).  Kbar, read only down its
  // columns, and the fp32 and d_k = 16 tiles stay row-major with a padded
  // row.
  static constexpr bool SWZ = std::is_same<E, Bf16>::value && DK % 32 == 0;
  static constexpr int LDK = SWZ ? DK + 16 : DK + S::M::PAD;  // row stride of K+, K-, Q+
  static constexpr int LDB = DK + S::M::PAD;                  // row stride of Kbar
  // element offset of (row r, channel c) in K+, K- or Q+
  static constexpr __host__ __device__ int at(int r, int c) {
    if constexpr (SWZ) {
      const int u = c >> 2, j = u & 7;  // 4-channel unit, its place in the k-step
      return r * LDK + 8 * (4 * (u >> 3) + (j & 3)) + 4 * (j >> 2) + (c & 3);
    } else {
      return r * LDK + c;
    }
  }
  // element offset of the operand fragment of row r, k-step s, lane group g
  static constexpr __host__ __device__ int frag_at(int r, int s, int g) { return r * LDK + 32 * s + 8 * g; }
  // every (row, channel) has its own element of the C x LDK tile, and each
  // fragment is the lane's channels in operand order
  static constexpr bool layout_ok() {
    if constexpr (!SWZ) {
      return true;
    } else {
      bool used[C * LDK] = {};
      for (int r = 0; r < C; ++r)
        for (int c = 0; c < DK; ++c) {
          const int o = at(r, c);
          if (o < r * LDK || o >= r * LDK + DK || used[o]) return false;
          used[o] = true;
        }
      for (int r = 0; r < C; ++r)
        for (int s = 0; s < DK / 32; ++s)
          for (int g = 0; g < 4; ++g)
            for (int e = 0; e < 4; ++e)
              if (frag_at(r, s, g) + e != at(r, 32 * s + 4 * g + e) ||
                  frag_at(r, s, g) + 4 + e != at(r, 32 * s + 16 + 4 * g + e))
                return false;
      return true;
    }
  }
  static_assert(layout_ok(), "operand-tile layout");
  static constexpr int LDF = C + 4;                 // fp32 C x C tiles (16-byte aligned rows)
  static constexpr int NPAIR = S::NT * (S::NT + 1) / 2;  // lower-triangular 16x16 tiles
  static constexpr int APW = (NPAIR + NW_PREP - 1) / NW_PREP;  // A tiles per wave
  static_assert(NRG * RPG == C && NCG * NRG <= NTH_PREP, "prologue map");
  // LDS plan (bytes).  Four C x DK operand tiles live from tile formation to
  // the end of the fragment stores.  The scan scratch is used before them,
  // Mf and Xf after them, so both reuse the same bytes.
  static constexpr int TILE = C * LDK * static_cast<int>(sizeof(lds_t));
  static constexpr int TILEB = C * LDB * static_cast<int>(sizeof(lds_t));
  static constexpr int MF = C * LDF * 4;
  static constexpr int SCAN = NRG * DK * 4;
  static constexpr int R_TILES = 3 * TILE + TILEB;
  static constexpr int R_AFTER = 2 * MF;
  static constexpr int REGION = ((R_TILES > R_AFTER ? R_TILES : R_AFTER) > SCAN
                                     ? (R_TILES > R_AFTER ? R_TILES : R_AFTER)
                                     : SCAN);
  static constexpr int OFF_KP = 0, OFF_KM = TILE, OFF_QP = 2 * TILE, OFF_KB = 3 * TILE;
  static constexpr int OFF_MF = 0, OFF_XF = MF, OFF_SCAN = 0;
  // Tm fragments are staged for a delayed write when they fit next to the
  // rest (two workgroups per CU); otherwise they are written directly.
  static constexpr int TMB = S::NTRI * S::FRAG;
  static constexpr bool STAGE_TM = REGION + 4 * DK + 4 * C + TMB <= 80 * 1024;
  struct Smem {
    alignas(16) char region[REGION];
    alignas(16) float gC[DK];
    alignas(16) float beta[C];
    alignas(16) char tm[STAGE_TM ? TMB : 16];
  };
};

// CHANNEL: per-channel gate (the KDA case), compiled without the gate-kind
// branches around the input loads; otherwise the gate kind is read at run time.
template <typename E, int DK, int C, bool CHANNEL>
__global__ __launch_bounds__(NTH_PREP, 2) void chunk_prep_kernel(
    const typename E::storage* __restrict__ q, const typename E::storage* __restrict__ k,
    const typename E::storage* __restrict__ alpha, const typename E::storage* __restrict__ beta,
    char* __restrict__ ws, int T, int H, int n0, int nchunk, int ntask, int gate, int rule,
    int fused, float gscale) {
  using S = Shape<E, DK, C>;
  using P = PrepCfg<E, DK, C>;
  using M = typename S::M;
  using lds_t = typename S::lds_t;
  using frag = typename S::frag;
  using St = typename E::storage;
  if constexpr (CHANNEL) gate = kGateChannel;
  __shared__ typename P::Smem sm;
  lds_t* const Kp = reinterpret_cast<lds_t*>(sm.region + P::OFF_KP);
  lds_t* const Km = reinterpret_cast<lds_t*>(sm.region + P::OFF_KM);
  lds_t* const Qp = reinterpret_cast<lds_t*>(sm.region + P::OFF_QP);
  lds_t* const Kb = reinterpret_cast<lds_t*>(sm.region + P::OFF_KB);
  float* const Mf = reinterpret_cast<float*>(sm.region + P::OFF_MF);
  float* const Xf = reinterpret_cast<float*>(sm.region + P::OFF_XF);
  float* const scan = reinterpret_cast<float*>(sm.region + P::OFF_SCAN);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int cg = tid % P::NCG, rg = tid / P::NCG;
  const bool pro = rg < P::NRG;
  const int ch0 = 8 * cg;
  // this thread's eight channels of row r of K+, K- or Q+: two 8-byte
  // stores, the upper four channels first for channels 64 .. 127 (the order
  // that keeps a row's stores free of bank conflicts)
  const bool hi_first = P::SWZ && ((ch0 >> 6) & 1);
  const int o_first = P::at(0, hi_first ? ch0 + 4 : ch0), o_second = P::at(0, hi_first ? ch0 : ch0 + 4);
  // The per-thread fp32 scratch of eight channels (the decay scan, the
  // chunk's decay) is stored and read as two 16-byte halves, in the order
  // that keeps the accesses of a wave free of bank conflicts at d_k = 64, 128.
  const bool hswap = ((cg >> 2) ^ (cg >> 3)) & 1;
  auto put_halves = [&](float* p, f32x8 x) {
    const f32x4 lo = __builtin_shufflevector(x, x, 0, 1, 2, 3), hi = __builtin_shufflevector(x, x, 4, 5, 6, 7);
    *reinterpret_cast<f32x4*>(p + (hswap ? 4 : 0)) = hswap ? hi : lo;
    *reinterpret_cast<f32x4*>(p + (hswap ? 0 : 4)) = hswap ? lo : hi;
  };
  auto get_halves = [&](const float* p) -> f32x8 {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p + (hswap ? 4 : 0));
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + (hswap ? 0 : 4));
    return hswap ? __builtin_shufflevector(b, a, 0, 1, 2, 3, 4, 5, 6, 7)
                 : __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto put8 = [&](lds_t* tile, int r, f32x8 x) {
    if constexpr (P::SWZ) {
      const f32x4 lo = __builtin_shufflevector(x, x, 0, 1, 2, 3), hi = __builtin_shufflevector(x, x, 4, 5, 6, 7);
      M::store4(&tile[r * P::LDK + o_first], hi_first ? hi : lo);
      M::store4(&tile[r * P::LDK + o_second], hi_first ? lo : hi);
    } else {
      M::store8(&tile[r * P::LDK + ch0], x);
    }
  };
  // this lane's operand fragment of row r, k-step s2 of K+, K- or Q+
  auto opnd = [&](const lds_t* tile, int r, int s2) -> frag {
    if constexpr (P::SWZ) {
      return *reinterpret_cast<const frag*>(tile + P::frag_at(r, s2, g));
    } else {
      const lds_t* row = tile + r * P::LDK;
      const int kb = 32 * s2 + 4 * g;
      return (S::KODD && s2 == S::NKS - 1) ? M::half(row + kb) : M::pair(row + kb, row + kb + 16);
    }
  };

  // Token row of (task, r), clamped into the sequence so loads stay in bounds.
  // This launch covers chunks n0 .. n0 + nchunk - 1 of every chain.  Tasks
  // are chunk-major (task = (n - n0) * nchain + chain), so the workspace
  // holds chunk n of every chain in one contiguous run, which the state pass
  // reads at its step n.
  const int nchain = ntask / nchunk;
  const long nrow = static_cast<long>(nchain) * T;  // token rows of every input tensor
  auto rowptr = [&](int task, int r) -> long {
    const int nl = task / nchain, chain = task - nl * nchain, n = n0 + nl;
    const int b = chain / H, h = chain - b * H;
    const int t = min(n * C + r, T - 1);
    return (static_cast<long>(b) * T + t) * H + h;
  };

  // a slot store of `bytes` at offset off of a task's slot
  auto slot_ok = [&](const char* sl, long off, int bytes) {
    return chk_ok((sl - ws) + off, static_cast<long>(ntask) * S::SLOT, kSiteSlotStore, bytes) &&
           chk_ok(off, S::SLOT, kSiteSlotStore, bytes);
  };

  Raw8<St> ra[P::RPG], rk[P::RPG], rq[P::RPG];
  St rb = St(0);
  auto prefetch = [&](int task) {
    if (task < ntask) {
      if (pro) {
#pragma unroll
        for (int rr = 0; rr < P::RPG; ++rr) {
          const long row = rowptr(task, rg * P::RPG + rr);
          if (gate == kGateChannel)
            ra[rr].load(alpha + chk(row * DK + ch0, nrow * DK, kSiteAlpha, 8));
          else if (gate == kGateHead)
            ra[rr].load_one(alpha + chk(row, nrow, kSiteAlpha));  // one decay for every channel of the head
          else
            ra[rr].ones();
          rk[rr].load(k + chk(row * DK + ch0, nrow * DK, kSiteQK, 8));
          rq[rr].load(q + chk(row * DK + ch0, nrow * DK, kSiteQK, 8));
        }
      }
      if (tid < C) rb = beta[chk(rowptr(task, tid), nrow, kSiteBeta)];
    }
  };
  prefetch(blockIdx.x);

  // The Tm fragments of a task are staged in LDS and written out early in
  // the next task, right behind the other stores: a wave's loads and stores
  // retire in issue order, so a store issued at the very end of a task would
  // hold up the next task's first use of its prefetched inputs.
  char* tm_slot = nullptr;  // slot whose Tm fragments are staged
  auto flush_tm = [&]() {
    if (P::STAGE_TM && tm_slot != nullptr) {
      // the lane offset (lane * fragment bytes per lane) is recomputed here
      // rather than kept live across tasks
      static_assert(S::FB == 16 || S::FB == 32, "lane fragment bytes");
      uint32_t lo;
      asm volatile("v_lshlrev_b32 %0, %2, %1" : "=v"(lo) : "v"(lane), "i"(S::FB == 16 ? 4 : 5));
      for (int i = wave; i < S::NTRI; i += NW_PREP)
        if (slot_ok(tm_slot, S::OFF_TM + i * S::FRAG + lo, S::FB))
          __builtin_nontemporal_store(*reinterpret_cast<const frag*>(sm.tm + i * S::FRAG + lo),
                                      reinterpret_cast<frag*>(tm_slot + S::OFF_TM + i * S::FRAG + lo));
    }
  };

  for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
    const int n = n0 + task / nchain;
    const int valid = min(C, T - n * C);
    char* slot = ws + static_cast<long>(task) * S::SLOT;

    // ---- 1. decay scan, from the prefetched registers
    f32x8 lg[P::RPG];
    __syncthreads();  // the previous task is done with every LDS byte
    if (pro) {
      f32x8 run;
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] = 1.f;
#pragma unroll
      for (int rr = 0; rr < P::RPG; ++rr) {
        const bool ok = rg * P::RPG + rr < valid;
        f32x8 a = gate == kGateHead ? ra[rr].unpack_one() : ra[rr].unpack();
        if (fused && gate != kGateNone) {  // raw gate projection -> decay
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = gate_map(a[e], gscale);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] *= ok ? a[e] : 1.f;
        lg[rr] = run;
      }
      put_halves(&scan[rg * DK + ch0], run);
    }
    if (tid < C) {
      const float bx = load_scalar(&rb, 0);
      sm.beta[tid] = tid < valid ? (fused ? sigmoid_f(bx) : bx) : 0.f;
    }

    __syncthreads();
    // The tiles below divide by the cumulative decay gamma_r, which must stay
    // in the normal fp32 range.  With alpha in (0, 1] gamma_r falls with r,
    // so the chunk's whole decay gamma_C decides: a chunk with gamma_C below
    // 2^-126 in some channel (an alpha of 0, or a product over the chunk
    // below about e^-87) is outside the chunked form's domain.  It is flagged
    // and gets NaN write strengths (Tm), so its outputs, the state and all
    // later outputs of the chain come out NaN instead of silently wrong.
    if (tid < DK) {  // exclusive products of the row-group totals, per channel
      float tot[P::NRG];
#pragma unroll
      for (int gg = 0; gg < P::NRG; ++gg) tot[gg] = scan[gg * DK + tid];
      float p = 1.f;
#pragma unroll
      for (int gg = 0; gg < P::NRG; ++gg) {
        scan[gg * DK + tid] = p;
        p *= tot[gg];
      }
      sm.gC[tid] = p;
      if (!(p >= 0x1p-126f)) {
        // beta = NaN makes Tm = X Diag(beta) NaN (beta is next read after
        // phase 3; every thread that finds the chunk out of range writes
        // the same values)
        const float nan = __builtin_nanf("");
        for (int i = 0; i < C; i += 4) *reinterpret_cast<f32x4*>(&sm.beta[i]) = f32x4{nan, nan, nan, nan};
      }
    }
    __syncthreads();
    f32x8 pre, gc;
    if (pro) {
      pre = get_halves(&scan[rg * DK + ch0]);
      gc = get_halves(&sm.gC[ch0]);
    }
    __syncthreads();  // the scan scratch is about to be overwritten by the tiles

    // ---- 2. decay-scaled operand tiles [r][channel] (layout: PrepCfg)
    if (pro) {
#pragma unroll
      for (int rr = 0; rr < P::RPG; ++rr) {
        const int r = rg * P::RPG + rr;
        const bool ok = r < valid;  // rows past the sequence: k = q = 0
        f32x8 kk = rk[rr].unpack(), qq = rq[rr].unpack();
        if (fused) {
          // L2-normalise the token's key and query: the NCG threads of a row
          // hold its channels in 8-wide groups (adjacent lanes).
          float sk = 0.f, sq = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) { sk += kk[e] * kk[e]; sq += qq[e] * qq[e]; }
#pragma unroll
          for (int off = 1; off < P::NCG; off <<= 1) {
            sk += __shfl_xor(sk, off);
            sq += __shfl_xor(sq, off);
          }
          const float ik = sk > 0.f ? rsqrtf(sk) : 0.f, iq = sq > 0.f ? rsqrtf(sq) : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) { kk[e] *= ik; qq[e] *= iq; }
        }
        f32x8 kp, qp, km, kb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gam = lg[rr][e] * pre[e];
          const float inv = __builtin_amdgcn_rcpf(gam);
          const float kv = ok ? kk[e] : 0.f, qv = ok ? qq[e] : 0.f;
          kp[e] = kv * gam;
          qp[e] = qv * gam;
          km[e] = kv * inv;
          kb[e] = km[e] * gc[e];
        }
        put8(Kp, r, kp);
        put8(Qp, r, qp);
        put8(Km, r, km);
        M::store8(&Kb[r * P::LDB + ch0], kb);
      }
    }
    __syncthreads();

    // ---- 3. Gram tiles (kept in registers), P fragments, and the K+ / Q+ /
    //         Kbar^T fragments copied into the workspace slot; first the
    //         previous task's Tm fragments.  This task's inputs are all in
    //         use by now: saying so here keeps the compiler from waiting on
    //         this task's stores before the next prefetch reuses registers.
    __builtin_amdgcn_s_waitcnt(0);
    flush_tm();
    f32x4 Aacc[P::APW];
    {
      int job = 0;
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int tc = 0; tc <= tr; ++tc, ++job) {
          if (job % NW_PREP != wave) continue;
          frag af[S::NKS], bf[S::NKS];
#pragma unroll
          for (int s2 = 0; s2 < S::NKS; ++s2) {
            af[s2] = opnd(Kp, 16 * tr + c16, s2);
            bf[s2] = opnd(Km, 16 * tc + c16, s2);
          }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < S::NKS; ++s2) acc = M::mma(af[s2], bf[s2], acc);
          Aacc[job / NW_PREP] = acc;  // job % NW_PREP == wave
        }
      job = 0;
      // P fragments (tr, s), s <= tr/2, from P^T tiles: the accumulator of
      // the product K- Q+^T holds P[16tr+c16][16tc+4g+e] in lane (g, c16),
      // i.e. exactly the operand order.
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int s2 = 0; s2 <= tr / 2; ++s2, ++job) {
          if ((job + 1) % NW_PREP != wave) continue;
          f32x4 half_acc[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int tc = 2 * s2 + hh;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (tc <= tr) {
              frag af[S::NKS], bf[S::NKS];
#pragma unroll
              for (int ks = 0; ks < S::NKS; ++ks) {
                af[ks] = opnd(Km, 16 * tc + c16, ks);
                bf[ks] = opnd(Qp, 16 * tr + c16, ks);
              }
#pragma unroll
              for (int ks = 0; ks < S::NKS; ++ks) acc = M::mma(af[ks], bf[ks], acc);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (16 * tc + 4 * g + e > 16 * tr + c16) acc[e] = 0.f;
            }
            half_acc[hh] = acc;
          }
          frag* dst = reinterpret_cast<frag*>(slot + S::OFF_PP + (S::tri(tr) + s2) * S::FRAG);
          if (slot_ok(slot, S::OFF_PP + (S::tri(tr) + s2) * S::FRAG + lane * S::FB, S::FB))
            __builtin_nontemporal_store(M::from_acc(half_acc[0], half_acc[1]), &dst[lane]);
        }
      // K+ and Q+ fragments: rows r, k = channels.
      constexpr int NKQ = 2 * S::NT * S::NKS;
      for (int jj = wave; jj < NKQ; jj += NW_PREP) {
        const int w2 = jj & 1, ts = jj >> 1;  // ts = t * NKS + s
        const int t = ts / S::NKS, s2 = ts - t * S::NKS;
        const frag f = opnd(w2 ? Qp : Kp, 16 * t + c16, s2);
        if (slot_ok(slot, (w2 ? S::OFF_QP : S::OFF_KP) + ts * S::FRAG + lane * S::FB, S::FB))
          __builtin_nontemporal_store(f, &reinterpret_cast<frag*>(slot + (w2 ? S::OFF_QP : S::OFF_KP) + ts * S::FRAG)[lane]);
      }
      // Kbar^T fragments: rows = channels 16t + c16, k = token rows, gathered
      // down a column of the row-major Kbar tile.
      constexpr int NKB = S::NTK * S::NCS;
      for (int jj = wave; jj < NKB; jj += NW_PREP) {
        const int t = jj / S::NCS, s2 = jj - t * S::NCS;
        const int col = 16 * t + c16;
        const int r0 = 32 * s2 + 4 * g;
        frag f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = Kb[(r0 + e) * P::LDB + col];
        if (S::CODD && s2 == S::NCS - 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) f[4 + e] = M::cvt(0.f);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) f[4 + e] = Kb[(r0 + 16 + e) * P::LDB + col];
        }
        if (slot_ok(slot, S::OFF_KB + jj * S::FRAG + lane * S::FB, S::FB))
          __builtin_nontemporal_store(f, &reinterpret_cast<frag*>(slot + S::OFF_KB + jj * S::FRAG)[lane]);
      }
      if (tid < DK && slot_ok(slot, S::OFF_GC + 4 * tid, 4))
        reinterpret_cast<float*>(slot + S::OFF_GC)[tid] = sm.gC[tid];
    }
    __syncthreads();  // the operand tiles are dead: Mf and Xf take their bytes
    // The next task's inputs load while this one finishes.  Issued after
    // this task's stores and before none, so the next task's first use of
    // them waits only for stores that are long done.
    prefetch(task + gridDim.x);

    // ---- 4. Mf = Diag(beta) strict_lower(A), then X = (I + Mf)^{-1}
    {
      int job = 0;
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int tc = 0; tc <= tr; ++tc, ++job) {
          if (job % NW_PREP != wave) continue;
          const f32x4 acc = Aacc[job / NW_PREP];
          const int jc = 16 * tc + c16;
          const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * tr + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * tr + 4 * g + e;
            // without the correction there is no erase term: A = 0, Tm = Diag(beta)
            Mf[r * P::LDF + jc] = jc < r && rule == kRuleDelta ? bt[e] * acc[e] : 0.f;
          }
        }
    }
    __syncthreads();
    // diagonal 16x16 blocks by substitution, one wave per block
    for (int bi = wave; bi < S::NT; bi += NW_PREP) {
      if (lane < 16) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* mrow = &Mf[(16 * bi + r) * P::LDF + 16 * bi];
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
        for (int r = 0; r < 16; ++r) Xf[(16 * bi + r) * P::LDF + 16 * bi + lane] = x[r];
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
          for (int s2 = 0; s2 < 4; ++s2) {
            av[s2] = Mf[(16 * aa + c16) * P::LDF + 16 * cc + 4 * s2 + g];
            bv[s2] = Xf[(16 * cc + 4 * s2 + g) * P::LDF + 16 * bb + c16];
          }
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) y = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s2], bv[s2], y, 0, 0, 0);
        }
        float av[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) av[s2] = Xf[(16 * aa + c16) * P::LDF + 16 * aa + 4 * g + s2];
        f32x4 xo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) xo = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s2], y[s2], xo, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Xf[(16 * aa + 4 * g + e) * P::LDF + 16 * bb + c16] = -xo[e];
      }
    }
    __syncthreads();

    // ---- 5. Tm = X Diag(beta) fragments (rows r, k = columns), s <= tr/2.
    //         X is lower triangular: entries above the diagonal are masked.
    {
      int job = 0;
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int s2 = 0; s2 <= tr / 2; ++s2, ++job) {
          if (job % NW_PREP != wave) continue;
          const int r = 16 * tr + c16;
          const float* xrow = Xf + r * P::LDF;
          const int kb = 32 * s2 + 4 * g;
          f32x8 t8;
          const f32x4 lo = *reinterpret_cast<const f32x4*>(xrow + kb);
#pragma unroll
          for (int e = 0; e < 4; ++e) t8[e] = kb + e <= r ? lo[e] * sm.beta[kb + e] : 0.f;
          if (S::CODD && s2 == S::NCS - 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) t8[4 + e] = 0.f;
          } else {
            const f32x4 hi = *reinterpret_cast<const f32x4*>(xrow + kb + 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) t8[4 + e] = kb + 16 + e <= r ? hi[e] * sm.beta[kb + 16 + e] : 0.f;
          }
          if constexpr (P::STAGE_TM)
            reinterpret_cast<frag*>(sm.tm + (S::tri(tr) + s2) * S::FRAG)[lane] = M::from8(t8);
          else if (slot_ok(slot, S::OFF_TM + (S::tri(tr) + s2) * S::FRAG + lane * S::FB, S::FB))
            __builtin_nontemporal_store(M::from8(t8), &reinterpret_cast<frag*>(slot + S::OFF_TM + (S::tri(tr) + s2) * S::FRAG)[lane]);
        }
    }
    tm_slot = slot;
  }
  if constexpr (P::STAGE_TM) {
    __syncthreads();  // the last task's Tm fragments are staged
    flush_tm();
  }
}

// ============================================================ state pass
constexpr size_t kLdsLimit = 160 * 1024;

template <typename E, int DK, int DVB, int C>
struct PassCfg {
  using S = Shape<E, DK, C>;
  static constexpr int NSLAB = DVB / 16;                 // 16-column state slabs
  // Two compute waves per slab: the state wave runs the sequential chain
  // (K+ S, Tm R, Kbar^T U) and hands the bf16 state and U to the output wave,
  // which forms O = Q+ S + P U next to it on another SIMD.
  static constexpr int NCW = 2 * NSLAB;
  static constexpr int NCP = 10 - NCW;                   // copy waves (loads)
  static constexpr int NTH = 64 * (NCW + NCP + 2);       // + one store wave, one prefetch wave
  // One workgroup per CU: its waves spread over the 4 SIMDs, so a SIMD holds
  // WPE of them and each may use 512 / WPE registers.
  static constexpr int WPE = (NTH / 64 + 3) / 4;
  static constexpr int SLOT = S::SLOT;
  static constexpr int ESZ = static_cast<int>(sizeof(typename E::storage));
  // Value / output tiles of one chunk: C rows x DVB columns, row-major,
  // copied one 1 KiB wave instruction at a time (the last may run past row
  // C into the tile's padding).
  static constexpr int VROW = DVB * ESZ;                 // bytes per tile row
  static constexpr int LPR = VROW / 16;                  // 16-byte lanes per row
  static constexpr int RPI = 64 / LPR;                   // rows per wave instruction
  static constexpr int NVI = (C + RPI - 1) / RPI;        // instructions per tile
  static constexpr int VTILE = NVI * 1024;               // bytes per tile buffer
  // With two slabs, rows with bit 2 set swap their two slab halves in LDS:
  // (row r, 16-byte piece k) sits at 16-byte position r * LPR + (k ^ VSW)
  // for those rows, r * LPR + k otherwise.  The compute waves read values and
  // write outputs down columns, lane groups four rows apart; without the swap
  // those rows share LDS banks (one extra cycle per half wave).  For a wave,
  // the swap is the same for every row it touches, so its addresses keep one
  // base.  One-slab tiles are left as they are.
  static constexpr int VSW = NSLAB == 2 ? LPR / 2 : 0;
  static_assert(RPI % 8 == 0, "the swap keeps rows in their 1 KiB copy unit");
  static constexpr __host__ __device__ int vidx(int r, int c) {  // element index of (row r, column c)
    return ((r * LPR + (((c * ESZ) / 16) ^ (VSW * ((r >> 2) & 1)))) * 16 + (c * ESZ) % 16) / ESZ;
  }
  static_assert(VROW % 16 == 0 && 64 % LPR == 0 && NSLAB <= 2, "pass map");
  // Hand-over areas: the state operand S (NKS fragments per slab, double
  // buffered: written at the end of chunk n for chunk n + 1), U (NCS
  // fragments per slab) and one ready counter per slab.
  static constexpr int XS = NSLAB * S::NKS * S::FRAG;
  static constexpr int XU = NSLAB * S::NCS * S::FRAG;
  static constexpr int REST = 4 * VTILE + 1024 + 2 * XS + XU + 64;
  // Double-buffer the slot when two fit next to everything else.
  static constexpr int NBUF = 2 * static_cast<size_t>(SLOT) + REST <= kLdsLimit ? 2 : 1;
  static constexpr int OFF_V = NBUF * SLOT;
  static constexpr int OFF_O = OFF_V + 2 * VTILE;
  static constexpr int OFF_SINK = OFF_O + 2 * VTILE;     // 1 KiB the prefetch loads land in
  static constexpr int OFF_XS = OFF_SINK + 1024;
  static constexpr int OFF_XU = OFF_XS + 2 * XS;
  static constexpr int OFF_FLAG = OFF_XU + XU;
  static constexpr size_t smem_bytes = static_cast<size_t>(OFF_FLAG) + 64;
};

// One workgroup per (batch, head, block of DVB value columns), over chunks
// n0 .. n0 + nchunk - 1 of the sequence (a segment; the whole sequence when
// it fits the workspace).  Inside the kernel n counts chunks from n0: slot n
// of the workspace, buffer parities and the hand-over counters all use it;
// token rows are (n0 + n) * C + r.  S0 is the state entering chunk n0 (NULL:
// zero), ST receives the state after the last chunk (NULL: not stored).  Each
// 16-column slab of the fp32 state has a state wave, which keeps the slab in
// accumulator registers and runs the sequential chain, and an output wave on
// another SIMD, which forms the slab's output from the state and U the state
// wave hands over in LDS.  Copy waves move the workspace slot and the value
// tile into LDS, a store wave writes the output tile out of it, and a
// prefetch wave pulls later slots into L2.  Value and output tiles are
// double-buffered, the slot too when it fits, so one barrier per chunk
// suffices:
//   [A] slot n and values n are in LDS, output n-1 is complete in LDS, the
//       state operand entering chunk n is in its hand-over buffer
//   copy: start slot n+1 and values n+1, wait for them
//   store: read output n-1 from LDS, issue its global stores (never waited
//          on inside the loop; drained once before the wave ends)
//   state: R = V - K+ S, U = Tm R, publish U, S <- gamma_C S + Kbar^T U,
//          publish the next state operand
//   output: O = Q+ S (before U is ready), then + P U, into the output tile
// DELTA: the error-correcting write (R = V - K+ S); without it R = V.  A
// template parameter, so that each kernel holds one chain loop.
template <typename E, int DK, int DVB, int C, bool DELTA>
__global__ __launch_bounds__((PassCfg<E, DK, DVB, C>::NTH))
__attribute__((amdgpu_waves_per_eu(PassCfg<E, DK, DVB, C>::WPE, PassCfg<E, DK, DVB, C>::WPE))) void state_pass_kernel(
    const char* __restrict__ ws, const typename E::storage* __restrict__ v,
    const float* __restrict__ S0, typename E::storage* __restrict__ o, float* __restrict__ ST,
    int T, int H, int DV, int n0, int nchunk, int wait_limit) {
  using S = Shape<E, DK, C>;
  using K = PassCfg<E, DK, DVB, C>;
  using M = typename S::M;
  using frag = typename S::frag;
  using St = typename E::storage;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int chain = blockIdx.x, vb = blockIdx.y;
  const int b = chain / H, h = chain - b * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool copier = wave >= K::NCW && wave < K::NCW + K::NCP;
  const bool storer = wave == K::NCW + K::NCP;
  const int cw = wave - K::NCW;  // copy-wave index
  const long rs = static_cast<long>(H) * DV;  // element stride between tokens
  const long base = static_cast<long>(b) * T * rs + static_cast<long>(h) * DV + vb * DVB;
  // extents for the checked build: this launch's slots (bytes), v and o
  // (elements: B * H = gridDim.x chains), S0 and S_T (elements)
  const long nslot = static_cast<long>(nchunk) * gridDim.x * K::SLOT;
  const long nval = static_cast<long>(gridDim.x) * T * DV;
  const long nstate = static_cast<long>(gridDim.x) * DK * DV;
  constexpr int VE = 16 / K::ESZ;  // elements per 16-byte lane access
  auto lds_ok = [&](long off) { return chk_ok(off, static_cast<long>(K::smem_bytes), kSiteLds, 1024); };

  // ------------------------------------------------------------ copy waves
  // the tile row and 16-byte piece this lane moves (position lane of a copy unit)
  const int crow = lane / K::LPR, cbyte = 16 * ((lane % K::LPR) ^ (K::VSW * ((crow >> 2) & 1)));
  auto stage_slot = [&](int n, int buf) {
    const long s0 = (static_cast<long>(n) * gridDim.x + chain) * K::SLOT;
    for (int u = cw; u < K::SLOT / 1024; u += K::NCP) {
      const long off = chk(s0 + u * 1024 + lane * 16, nslot, kSiteSlotLoad, 16);
      if (lds_ok(buf * K::SLOT + u * 1024))
        __builtin_amdgcn_global_load_lds((gvoid_t*)(ws + off), (lvoid_t*)(lds + buf * K::SLOT + u * 1024), 16, 0, 0);
    }
  };
  auto stage_v = [&](int n) {
    const int vo = K::OFF_V + (n & 1) * K::VTILE;
    for (int u = cw; u < K::NVI; u += K::NCP) {
      const int t = min((n0 + n) * C + u * K::RPI + crow, T - 1);  // rows past T: zeroed at use
      const long e = chk(base + t * rs + cbyte / K::ESZ, nval, kSiteValue, VE);
      if (lds_ok(vo + u * 1024))
        __builtin_amdgcn_global_load_lds((gvoid_t*)(v + e), (lvoid_t*)(lds + vo + u * 1024), 16, 0, 0);
    }
  };
  // Prefetch wave: pulls its share of chunk n's slot (the value blocks of a
  // chain split the slot units between them) and its own value rows into
  // L2, so that the copy waves' loads for that chunk hit there.  Each load is
  // a whole 1 KiB unit (partial-line touches do not fill the line); the data
  // lands in a 1 KiB LDS sink that is never read.
  const int qu = (K::SLOT / 1024 + gridDim.y - 1) / gridDim.y;
  auto prefetch = [&](int n) {
    const long s0 = (static_cast<long>(n) * gridDim.x + chain) * K::SLOT;
    char* sink = lds + K::OFF_SINK;
    for (int i = 0; i < qu; ++i) {
      const int u = min(vb * qu + i, K::SLOT / 1024 - 1);
      const long off = chk(s0 + u * 1024 + lane * 16, nslot, kSitePrefetch, 16);
      __builtin_amdgcn_global_load_lds((gvoid_t*)(ws + off), (lvoid_t*)sink, 16, 0, 0);
    }
    for (int u = 0; u < K::NVI; ++u) {
      const int t = min((n0 + n) * C + u * K::RPI + crow, T - 1);
      const long e = chk(base + t * rs + cbyte / K::ESZ, nval, kSiteValue, VE);
      __builtin_amdgcn_global_load_lds((gvoid_t*)(v + e), (lvoid_t*)sink, 16, 0, 0);
    }
  };
  // The compiler makes any LDS read wait for every earlier global access of
  // the wave (it cannot tell this wave's stores from the copy waves' LDS-DMA
  // loads), which would hold this wave at each chunk until the previous
  // chunk's stores are acknowledged.  The reads are therefore written out
  // with their own LDS wait; the data was published by the barrier before.
  auto store_out = [&](int n) {
    const uint32_t src = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) char*)(lds + K::OFF_O + (n & 1) * K::VTILE + lane * 16)));
    uint4 x[K::NVI];
#pragma unroll
    for (int u = 0; u < K::NVI; ++u) {
      u32x4 y;
      asm volatile("ds_read_b128 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)" : "=v"(y) : "v"(src), "i"(u * 1024) : "memory");
      x[u] = uint4{y[0], y[1], y[2], y[3]};
    }
#pragma unroll
    for (int u = 0; u < K::NVI; ++u) {
      const int r = u * K::RPI + crow, t = (n0 + n) * C + r;
      if (r < C && t < T && chk_ok(base + t * rs + cbyte / K::ESZ, nval, kSiteOut, VE))
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(o + base + t * rs) + cbyte) = x[u];
    }
  };

  // --------------------------------------------------------- compute waves
  // State wave of slab j (wave j) holds Sa[ti] = S[16 ti + 4 g + e][col] in
  // accumulator registers; output wave of slab j is wave NSLAB + j.
  const int c16 = lane & 15, g = lane >> 4;
  const bool stater = wave < K::NSLAB, outer = !stater && wave < K::NCW;
  const int slab = stater ? wave : wave - K::NSLAB;
  const int col = vb * DVB + 16 * slab + c16;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  frag* xs = reinterpret_cast<frag*>(lds + K::OFF_XS) + slab * S::NKS * 64;  // + buffer * XS/FRAG*64
  frag* xu = reinterpret_cast<frag*>(lds + K::OFF_XU) + slab * S::NCS * 64;
  int* flag = reinterpret_cast<int*>(lds + K::OFF_FLAG) + slab;
  constexpr int XSF = K::XS / S::FRAG * 64;  // frag elements per state buffer
  auto slot_of = [&](int n) -> const char* { return lds + (K::NBUF == 2 ? (n & 1) : 0) * K::SLOT; };

  // Each role runs its own loop over the chunks, so the register allocator
  // sees one role's values at a time.  Every wave passes the same workgroup
  // barriers in the same order: [A] at the top of each chunk, [B] after the
  // compute waves are done with a single slot buffer (only when the slot is
  // not double-buffered), and one final [A].  The store and prefetch waves
  // pass them without draining their memory operations: nothing in the
  // workgroup waits on those.
  if (stater) {
    f32x4 Sa[S::NTK];
    frag sfr[S::NKS];  // bf16 (or fp32) operand copy of the state entering the chunk
    if (S0 != nullptr) {
      const long s0 = (static_cast<long>(chain) * DK + 4 * g) * DV + col;
#pragma unroll
      for (int ti = 0; ti < S::NTK; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sa[ti][e] = S0[chk(s0 + (16 * ti + e) * DV, nstate, kSiteS0)];
    } else {
#pragma unroll
      for (int ti = 0; ti < S::NTK; ++ti) Sa[ti] = z;
    }
#pragma unroll
    for (int s2 = 0; s2 < S::NKS; ++s2) {
      sfr[s2] = M::from_acc(Sa[2 * s2], (S::KODD && s2 == S::NKS - 1) ? z : Sa[2 * s2 + 1]);
      xs[s2 * 64 + lane] = sfr[s2];
    }
    if (lane == 0) *flag = 0;

    // One chunk of the chain, straight-line per update rule.  For bf16 at
    // d_k = 128, C = 64 the operand reads of each product group go out as
    // one batch with a single LDS wait (see lds_read16).
    constexpr bool FAST = std::is_same<E, Bf16>::value && S::NT * S::NKS == 16 && S::NTRI == 6 &&
                          S::NTK == 8 && S::NTK * S::NCS == 16 && S::FRAG == 1024;
    auto chain_step = [&](int n) {
      const int t0 = (n0 + n) * C;
      const char* sl = slot_of(n);
      auto fr = [&](int off, int idx) -> frag {
        return reinterpret_cast<const frag*>(sl + off + idx * S::FRAG)[lane];
      };
      const uint32_t fb = lds_addr(sl) + 16 * lane, gb = lds_addr(sl) + 16 * g;
      const St* vt = reinterpret_cast<const St*>(lds + K::OFF_V + (n & 1) * K::VTILE);
      const float* gC = reinterpret_cast<const float*>(sl + S::OFF_GC);

      // R = V - K+ S  (R = V without the correction)
      f32x4 R[S::NT];
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr) R[tr] = z;
      if constexpr (DELTA) {
        frag akp[S::NT][S::NKS];
        if constexpr (FAST) {
          u32x4 r[16];
          lds_read16<S::OFF_KP, S::FRAG>(fb, r);
#pragma unroll
          for (int i = 0; i < 16; ++i) akp[i / S::NKS][i % S::NKS] = __builtin_bit_cast(frag, r[i]);
        } else {
#pragma unroll
          for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
            for (int s2 = 0; s2 < S::NKS; ++s2) akp[tr][s2] = fr(S::OFF_KP, tr * S::NKS + s2);
        }
        // the independent accumulator chains interleaved (k-step outermost)
#pragma unroll
        for (int s2 = 0; s2 < S::NKS; ++s2)
#pragma unroll
          for (int tr = 0; tr < S::NT; ++tr) R[tr] = M::mma(akp[tr][s2], sfr[s2], R[tr]);
      }
      frag atm[S::NTRI];
      f32x4 gcv[S::NTK];
      if constexpr (FAST) {
        u32x4 r[6], q[8];
        lds_read6_8<S::OFF_TM, S::FRAG, S::OFF_GC, 64>(fb, r, gb, q);
#pragma unroll
        for (int i = 0; i < 6; ++i) atm[i] = __builtin_bit_cast(frag, r[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) gcv[i] = __builtin_bit_cast(f32x4, q[i]);
      } else {
#pragma unroll
        for (int i = 0; i < S::NTRI; ++i) atm[i] = fr(S::OFF_TM, i);
#pragma unroll
        for (int ti = 0; ti < S::NTK; ++ti) gcv[ti] = *reinterpret_cast<const f32x4*>(gC + 16 * ti + 4 * g);
      }
      // Diag(gamma_C) S on the fp32 state (R used the operand copy of the
      // state entering the chunk); kept here so that gamma_C is dead before
      // the next operands arrive
#pragma unroll
      for (int ti = 0; ti < S::NTK; ++ti) {
        Sa[ti] *= gcv[ti];
        asm volatile("" : "+v"(Sa[ti]));
      }
      float vr[S::NT][4];
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[tr][e] = load_scalar(vt, K::vidx(16 * tr + 4 * g + e, 16 * slab + c16));
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) R[tr][e] = (t0 + 16 * tr + 4 * g + e < T ? vr[tr][e] : 0.f) - R[tr][e];
      frag rfr[S::NCS];
#pragma unroll
      for (int s2 = 0; s2 < S::NCS; ++s2)
        rfr[s2] = M::from_acc(R[2 * s2], (S::CODD && s2 == S::NCS - 1) ? z : R[2 * s2 + 1]);

      // U = Tm R  (Tm lower triangular: row tile tr uses k-steps s2 <= tr / 2)
      f32x4 U[S::NT];
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr) U[tr] = z;
#pragma unroll
      for (int s2 = 0; s2 < S::NCS; ++s2)
#pragma unroll
        for (int tr = 2 * s2; tr < S::NT; ++tr) U[tr] = M::mma(atm[S::tri(tr) + s2], rfr[s2], U[tr]);
      frag akb[S::NTK][S::NCS];
      if constexpr (FAST) {
        u32x4 r[16];
        lds_read16<S::OFF_KB, S::FRAG>(fb, r);
#pragma unroll
        for (int i = 0; i < 16; ++i) akb[i / S::NCS][i % S::NCS] = __builtin_bit_cast(frag, r[i]);
      } else {
#pragma unroll
        for (int ti = 0; ti < S::NTK; ++ti)
#pragma unroll
          for (int s2 = 0; s2 < S::NCS; ++s2) akb[ti][s2] = fr(S::OFF_KB, ti * S::NCS + s2);
      }
      frag ufr[S::NCS];
#pragma unroll
      for (int s2 = 0; s2 < S::NCS; ++s2) {
        ufr[s2] = M::from_acc(U[2 * s2], (S::CODD && s2 == S::NCS - 1) ? z : U[2 * s2 + 1]);
        xu[s2 * 64 + lane] = ufr[s2];
      }
      // publish U to the output wave: its LDS writes complete before the count
      if (lane == 0) __hip_atomic_store(flag, n + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);

      // S <- Diag(gamma_C) S + Kbar^T U
#pragma unroll
      for (int s2 = 0; s2 < S::NCS; ++s2)
#pragma unroll
        for (int ti = 0; ti < S::NTK; ++ti) Sa[ti] = M::mma(akb[ti][s2], ufr[s2], Sa[ti]);
      // the next chunk's state operand, for both waves of the slab
      frag* xn = xs + ((n + 1) & 1) * XSF;
#pragma unroll
      for (int s2 = 0; s2 < S::NKS; ++s2) {
        sfr[s2] = M::from_acc(Sa[2 * s2], (S::KODD && s2 == S::NKS - 1) ? z : Sa[2 * s2 + 1]);
        xn[s2 * 64 + lane] = sfr[s2];
      }
    };
    for (int n = 0; n < nchunk; ++n) {
      __syncthreads();  // [A]
      chain_step(n);
      if (K::NBUF == 1) __syncthreads();  // [B]
    }
    if (nchunk > 0) __syncthreads();  // final [A]
    if (ST != nullptr) {
      const long s0 = (static_cast<long>(chain) * DK + 4 * g) * DV + col;
#pragma unroll
      for (int ti = 0; ti < S::NTK; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (chk_ok(s0 + (16 * ti + e) * DV, nstate, kSiteST)) ST[s0 + (16 * ti + e) * DV] = Sa[ti][e];
    }
  } else if (outer) {
    // Output wave: O = Q+ S_in + P U into the output tile.
    for (int n = 0; n < nchunk; ++n) {
      __syncthreads();  // [A]
      const char* sl = slot_of(n);
      auto fr = [&](int off, int idx) -> frag {
        return reinterpret_cast<const frag*>(sl + off + idx * S::FRAG)[lane];
      };
      St* ot = reinterpret_cast<St*>(lds + K::OFF_O + (n & 1) * K::VTILE);
      const frag* xc = xs + (n & 1) * XSF;
      frag osf[S::NKS], aqp[S::NT][S::NKS];
#pragma unroll
      for (int s2 = 0; s2 < S::NKS; ++s2) osf[s2] = xc[s2 * 64 + lane];
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int s2 = 0; s2 < S::NKS; ++s2) aqp[tr][s2] = fr(S::OFF_QP, tr * S::NKS + s2);
      f32x4 O[S::NT];
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr) O[tr] = z;
#pragma unroll
      for (int s2 = 0; s2 < S::NKS; ++s2)
#pragma unroll
        for (int tr = 0; tr < S::NT; ++tr) O[tr] = M::mma(aqp[tr][s2], osf[s2], O[tr]);
      frag app[S::NTRI];
#pragma unroll
      for (int i = 0; i < S::NTRI; ++i) app[i] = fr(S::OFF_PP, i);
      // U of this chunk: the state wave publishes it part-way through the
      // chunk.  The wait is bounded (wait_limit polls; the state wave never
      // waits on this wave).  If it gives up, the chunk's output is NaN, so
      // the failure shows in the result instead of a stale U.
      bool ready = false;
      for (int it = 0; it < wait_limit; ++it) {
        if (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) > n) {
          ready = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      frag ufr[S::NCS];
#pragma unroll
      for (int s2 = 0; s2 < S::NCS; ++s2) ufr[s2] = xu[s2 * 64 + lane];
#pragma unroll
      for (int s2 = 0; s2 < S::NCS; ++s2)
#pragma unroll
        for (int tr = 2 * s2; tr < S::NT; ++tr) O[tr] = M::mma(app[S::tri(tr) + s2], ufr[s2], O[tr]);
      if (!ready) {
#pragma unroll
        for (int tr = 0; tr < S::NT; ++tr) O[tr] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      }
#pragma unroll
      for (int tr = 0; tr < S::NT; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) store_scalar(ot, K::vidx(16 * tr + 4 * g + e, 16 * slab + c16), O[tr][e]);
      if (K::NBUF == 1) __syncthreads();  // [B]
    }
    if (nchunk > 0) __syncthreads();  // final [A]
  } else if (copier) {
    if (nchunk > 0) {
      stage_slot(0, 0);
      stage_v(0);
      __builtin_amdgcn_s_waitcnt(0);
    }
    for (int n = 0; n < nchunk; ++n) {
      __syncthreads();  // [A]
      if (n + 1 < nchunk) {
        if (K::NBUF == 2) stage_slot(n + 1, (n + 1) & 1);
        stage_v(n + 1);
      }
      if (K::NBUF == 2) {
        __builtin_amdgcn_s_waitcnt(0);
      } else {
        __syncthreads();  // [B]: every compute wave is done with the single slot
        if (n + 1 < nchunk) stage_slot(n + 1, 0);
        __builtin_amdgcn_s_waitcnt(0);
      }
    }
    if (nchunk > 0) __syncthreads();  // final [A]
  } else if (storer) {
    for (int n = 0; n < nchunk; ++n) {
      __builtin_amdgcn_s_barrier();  // [A]
      if (n > 0) store_out(n - 1);   // its LDS reads complete before the stores issue
      if (K::NBUF == 1) __builtin_amdgcn_s_barrier();  // [B]
    }
    if (nchunk > 0) {
      __builtin_amdgcn_s_barrier();  // final [A]: the last output tile is in LDS
      store_out(nchunk - 1);
    }
    __builtin_amdgcn_s_waitcnt(0);
  } else {  // prefetch wave
    if (nchunk > 1) prefetch(1);
    for (int n = 0; n < nchunk; ++n) {
      __builtin_amdgcn_s_barrier();  // [A]
      if (n + 2 < nchunk) {
        __builtin_amdgcn_s_waitcnt(0);  // the previous chunk's prefetch has landed
        prefetch(n + 2);
      }
      if (K::NBUF == 1) __builtin_amdgcn_s_barrier();  // [B]
    }
    if (nchunk > 0) __builtin_amdgcn_s_barrier();  // final [A]
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// ================================================================== host

template <typename E, int DK, int C>
constexpr bool prep_fits() { return sizeof(typename PrepCfg<E, DK, C>::Smem) <= kLdsLimit / 2; }

// Value-block width of a state-pass workgroup: 32 columns (two compute
// waves), or 16 when d_v is 16.
constexpr int dvb_for(int dv) { return dv < 32 ? dv : 32; }

template <typename E, int DK, int DV, int C>
constexpr bool fits() {
  return prep_fits<E, DK, C>() && PassCfg<E, DK, dvb_for(DV), C>::smem_bytes <= kLdsLimit;
}

// CU count of the current device, cached per device (relaxed atomics: every
// thread that fills an entry writes the same value; devices past 63 are
// queried on every call; 256 if the query fails).
int num_cus() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool cached = dev >= 0 && dev < 64;
  if (cached) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (cached) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// State pass with value blocks of DVB columns: one workgroup per (chain,
// value block), over chunks n0 .. n0 + cnt - 1.
template <typename E, int DK, int DVB, int C, bool DELTA>
hipError_t launch_pass_rule(const PrefillArgs& a, const char* ws, int n0, int cnt,
                            const float* s_in, float* s_out) {
  using St = typename E::storage;
  using K = PassCfg<E, DK, DVB, C>;
  // Opt in to more than 64 KiB of LDS, once per device (bit d of the mask;
  // devices past 63 opt in on every launch).
  static std::atomic<unsigned long long> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit == 0 || !(attr_set.load(std::memory_order_acquire) & bit)) {
    const void* fn = reinterpret_cast<const void*>(&state_pass_kernel<E, DK, DVB, C, DELTA>);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(K::smem_bytes));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  // grid.x = (batch, head) chains, grid.y = value blocks: the value blocks
  // of one chain are gridDim.x apart in dispatch order, which keeps them on
  // one XCD (and its L2) whenever gridDim.x is a multiple of 8.
  hipLaunchKernelGGL((state_pass_kernel<E, DK, DVB, C, DELTA>), dim3(a.B * a.H, a.d_v / DVB),
                     dim3(K::NTH), K::smem_bytes, a.stream, ws, static_cast<const St*>(a.v),
                     s_in, static_cast<St*>(a.o), s_out, a.T, a.H, a.d_v, n0, cnt, wait_limit());
  return hipGetLastError();
}

template <typename E, int DK, int DVB, int C>
hipError_t launch_pass(const PrefillArgs& a, const char* ws, int n0, int cnt, const float* s_in,
                       float* s_out) {
  return a.rule == kRuleDelta ? launch_pass_rule<E, DK, DVB, C, true>(a, ws, n0, cnt, s_in, s_out)
                              : launch_pass_rule<E, DK, DVB, C, false>(a, ws, n0, cnt, s_in, s_out);
}

template <typename E, int DK, int C>
hipError_t launch_prep(const PrefillArgs& a, char* ws, int n0, int cnt) {
  using St = typename E::storage;
  const long ntask = static_cast<long>(a.B) * a.H * cnt;
  if (ntask == 0) return hipSuccess;
  // two resident workgroups per CU, each walking a strided list of chunks
  const int cus = num_cus();
  const int grid = static_cast<int>(ntask < 2 * cus ? ntask : 2 * cus);
  auto prep = a.gate == kGateChannel ? chunk_prep_kernel<E, DK, C, true> : chunk_prep_kernel<E, DK, C, false>;
  hipLaunchKernelGGL(prep, dim3(grid), dim3(NTH_PREP), 0, a.stream,
                     static_cast<const St*>(a.q), static_cast<const St*>(a.k),
                     static_cast<const St*>(a.alpha), static_cast<const St*>(a.beta), ws, a.T,
                     a.H, n0, cnt, static_cast<int>(ntask), a.gate, a.rule, a.fused ? 1 : 0,
                     a.gate_scale);
  return hipGetLastError();
}

template <typename E, int DK, int DV, int C>
hipError_t launch_t(const PrefillArgs& a) {
  const int nchunk = (a.T + C - 1) / C;
  const PrefillPlan p = prefill_plan(Shape<E, DK, C>::SLOT, static_cast<long>(a.B) * a.H, nchunk,
                                     DK, DV, a.ring_cap);
  if (a.workspace_bytes < p.total) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(a.workspace);
  // The state passes from segment to segment through S_T when the caller
  // wants it, else through the workspace's carrier area.
  float* carrier = a.S_T != nullptr ? a.S_T : reinterpret_cast<float*>(ws + p.carrier_off);
  // The chain of each value block is sequential over the chunks.  When the
  // 32-column blocks would leave more than half of the CUs idle (few long
  // sequences), 16-column blocks put twice as many chains of work on the
  // chip, each CU carrying one state slab instead of two.
  bool narrow = false;
  if constexpr (dvb_for(DV) == 32 && PassCfg<E, DK, 16, C>::smem_bytes <= kLdsLimit)
    narrow = static_cast<long>(a.B) * a.H * (DV / 32) * 2 <= num_cus();
  auto seg = [&](int i) { return std::make_pair(i * p.seg, min(p.seg, nchunk - i * p.seg)); };
  auto base = [&](int i) { return ws + static_cast<size_t>(i % p.nbuf) * p.half; };
  auto pass = [&](int i) -> hipError_t {
    const auto [n0, cnt] = seg(i);
    const float* s_in = i == 0 ? a.S0 : carrier;
    float* s_out = i == p.nseg - 1 ? a.S_T : carrier;
    if constexpr (dvb_for(DV) == 32 && PassCfg<E, DK, 16, C>::smem_bytes <= kLdsLimit) {
      if (narrow) return launch_pass<E, DK, 16, C>(a, base(i), n0, cnt, s_in, s_out);
    }
    return launch_pass<E, DK, dvb_for(DV), C>(a, base(i), n0, cnt, s_in, s_out);
  };
  auto prep = [&](int i) {
    const auto [n0, cnt] = seg(i);
    return launch_prep<E, DK, C>(a, base(i), n0, cnt);
  };

  for (int i = 0; i < p.nseg; ++i) {
    hipError_t e = prep(i);
    if (e != hipSuccess) return e;
    e = pass(i);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename E, int DK, int C>
hipError_t dispatch_dv(const PrefillArgs& a, size_t* slot) {
  switch (a.d_v) {
#define KDA_CASE(DV)                                                            \
  case DV:                                                                      \
    if constexpr (fits<E, DK, DV, C>()) {                                       \
      if (slot) { *slot = Shape<E, DK, C>::SLOT; return hipSuccess; }           \
      return launch_t<E, DK, DV, C>(a);                                         \
    } else {                                                                    \
      return hipErrorNotSupported;                                              \
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
hipError_t dispatch_c(const PrefillArgs& a, size_t* slot) {
  switch (a.chunk) {
    case 16: return dispatch_dv<E, DK, 16>(a, slot);
    case 32: return dispatch_dv<E, DK, 32>(a, slot);
    case 64: return dispatch_dv<E, DK, 64>(a, slot);
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

// --------------------------------------------- prefill without allocation
// Device memory of the allocation-free prefill: the segment ring (and the
// carrier state) live in this file-scope array, one copy per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel:
// it is a host-side stand-in, not a device address.  The address of each
// device's copy comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

// Per-device address of `scratch` (devices 0..63 cached; others looked up on
// every call).  The lookup runs with the device current.
hipError_t scratch_address(void** ptr) {
  static std::mutex mu;
  static void* cache[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      cache[dev] = p;
    }
    *ptr = cache[dev];
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  *ptr = p;
  return hipSuccess;
}

}  // namespace

bool noalloc_plan(size_t slot, long nchain, int nchunk, int d_k, int d_v, size_t* cap) {
  const size_t full = slot * static_cast<size_t>(nchain) * static_cast<size_t>(nchunk);
  if (full <= kNoAllocScratchBytes) {  // one segment, no carrier
    *cap = kNoAllocScratchBytes;
    return true;
  }
  const size_t carrier = static_cast<size_t>(nchain) * d_k * d_v * sizeof(float);
  if (carrier >= kNoAllocScratchBytes) return false;
  *cap = kNoAllocScratchBytes - carrier;
  return prefill_plan(slot, nchain, nchunk, d_k, d_v, *cap).total <= kNoAllocScratchBytes;
}

hipError_t launch_prefill_noalloc(const PrefillArgs& args) {
  PrefillArgs a = args;
  void* p = nullptr;
  hipError_t e = scratch_address(&p);
  if (e != hipSuccess) return e;
  a.workspace = p;
  a.workspace_bytes = kNoAllocScratchBytes;
  return launch_prefill(a);
}

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

namespace {
// Self-test of the checked build: one check of an index one past the end of
// a one-element extent; nothing is accessed.
__global__ void check_probe_kernel(long n) {
  if (threadIdx.x == 0) (void)chk(n, n, kSiteProbe);
}
}  // namespace

hipError_t launch_check_probe(hipStream_t stream) {
  hipLaunchKernelGGL(check_probe_kernel, dim3(1), dim3(64), 0, stream, 1L);
  return hipGetLastError();
}

unsigned prefill_check_take() { return check_take(); }

}  // namespace kda
