// C ABI of the KDA library: argument validation and kernel dispatch.
// The contract (layouts, ownership, errors) is documented in include/kda.h.
#include <stdint.h>

#include <atomic>

#include "../../include/kda.h"
#include "../../include/kda_testing.h"
#include "kda_check.h"
#include "kda_internal.h"

namespace kda {

namespace {
std::atomic<int> g_wait_limit{1 << 24};
std::atomic<size_t> g_ring_cap{kRingCap};
std::atomic<unsigned> g_check_sites_last{0};  // checked build: mask of the last failed call
}  // namespace

int wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
size_t ring_cap() { return g_ring_cap.load(std::memory_order_relaxed); }

int checked_finish(hipStream_t stream, int status) {
  if (!kChecked || status != KDA_OK) return status;
  if (hipStreamSynchronize(stream) != hipSuccess) return KDA_ERR_HIP;
  const unsigned m = prefill_check_take() | (decode_check_take() << 16) | (attnres_check_take() << 24);
  if (m == 0) return KDA_OK;
  g_check_sites_last.store(m, std::memory_order_relaxed);
  return KDA_ERR_CHECK;
}

}  // namespace kda

namespace {

constexpr int kVersion = 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool dtype_ok(int dt) { return dt == KDA_F32 || dt == KDA_BF16; }
bool gate_ok(int g) { return g == KDA_GATE_CHANNEL || g == KDA_GATE_HEAD || g == KDA_GATE_NONE; }
bool rule_ok(int r) { return r == KDA_RULE_DELTA || r == KDA_RULE_LINEAR; }
bool scale_ok(float c) { return c >= 0.f && c <= 3.0e38f; }  // finite, not negative (NaN fails)

int from_hip(hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  if (e == hipErrorNotSupported) return KDA_ERR_UNSUPPORTED;
  return KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_version(void) { return kVersion; }

int kda_testing_set_wait_limit(int polls) {
  if (polls < 0) return KDA_ERR_INVALID_ARG;
  kda::g_wait_limit.store(polls, std::memory_order_relaxed);
  return KDA_OK;
}

int kda_testing_wait_limit(void) { return kda::wait_limit(); }

int kda_testing_set_ring_cap(size_t bytes) {
  kda::g_ring_cap.store(bytes == 0 ? kda::kRingCap : bytes, std::memory_order_relaxed);
  return KDA_OK;
}

size_t kda_testing_ring_cap(void) { return kda::ring_cap(); }

int kda_testing_check_probe(void* stream) {
  try {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (kda::launch_check_probe(s) != hipSuccess) return KDA_ERR_HIP;
    return kda::checked_finish(s, KDA_OK);
  } catch (...) {
    return KDA_ERR_HIP;
  }
}

int kda_build_checked(void) { return kda::kChecked ? 1 : 0; }

unsigned int kda_check_sites(void) { return kda::g_check_sites_last.load(std::memory_order_relaxed); }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_CHECK: return "KDA_ERR_CHECK";
  }
  return "KDA_ERR_UNKNOWN";
}

size_t kda_fwd_chunked_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk,
                                       int dtype) {
  if (B < 1 || H < 1 || T < 0 || !dtype_ok(dtype) || !dim_ok(d_k) || !dim_ok(d_v)) return 0;
  size_t slot = 0;
  if (!kda::prefill_slot_bytes(dtype == KDA_BF16, d_k, d_v, chunk, &slot)) return 0;
  const long long nchunk = (static_cast<long long>(T) + chunk - 1) / chunk;
  if (static_cast<long long>(B) * H * nchunk > (1LL << 31) - 1) return 0;
  return kda::prefill_plan(slot, static_cast<long>(B) * H, static_cast<int>(nchunk), d_k, d_v,
                           kda::ring_cap())
      .total;
}

}  // extern "C"

namespace {

int fwd_impl(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
             const float* S0, void* o, float* S_T, int B, int T, int H, int d_k, int d_v,
             int chunk, int dtype, int gate, int rule, bool fused, float gate_scale,
             void* workspace, size_t workspace_bytes, void* stream, bool noalloc = false) {
  try {
    if (B < 1 || H < 1 || T < 0 || !dtype_ok(dtype) || !gate_ok(gate) || !rule_ok(rule) ||
        !scale_ok(gate_scale))
      return KDA_ERR_INVALID_ARG;
    if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
    if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
    const uintptr_t esz = dtype == KDA_BF16 ? 2 : 4;
    if (T > 0) {
      if (!q || !k || !v || !beta || !o || (gate != KDA_GATE_NONE && !alpha))
        return KDA_ERR_INVALID_ARG;
      if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return KDA_ERR_INVALID_ARG;
      // per-channel gates are read 16 bytes at a time; beta and per-head
      // gates one element at a time, so natural alignment is enough
      if (gate == KDA_GATE_CHANNEL && !aligned16(alpha)) return KDA_ERR_INVALID_ARG;
      if (gate == KDA_GATE_HEAD && reinterpret_cast<uintptr_t>(alpha) % esz != 0)
        return KDA_ERR_INVALID_ARG;
      if (reinterpret_cast<uintptr_t>(beta) % esz != 0) return KDA_ERR_INVALID_ARG;
    }
    if ((S0 && !aligned16(S0)) || (S_T && !aligned16(S_T))) return KDA_ERR_INVALID_ARG;
    // Token and state offsets are computed in 64-bit; keep grid sizes sane.
    if (static_cast<long long>(B) * H > (1LL << 31) - 1) return KDA_ERR_INVALID_ARG;
    if (!kda::prefill_supported(dtype == KDA_BF16, d_k, d_v, chunk)) return KDA_ERR_UNSUPPORTED;
    const long long nchunk = (static_cast<long long>(T) + chunk - 1) / chunk;
    if (static_cast<long long>(B) * H * nchunk > (1LL << 31) - 1) return KDA_ERR_INVALID_ARG;
    size_t slot = 0;
    kda::prefill_slot_bytes(dtype == KDA_BF16, d_k, d_v, chunk, &slot);
    size_t cap = 0;
    if (noalloc) {
      // the library's own device array must hold the whole plan
      if (!kda::noalloc_plan(slot, static_cast<long>(B) * H, static_cast<int>(nchunk), d_k, d_v,
                             &cap))
        return KDA_ERR_WORKSPACE;
    } else {
      // one reading of the ring budget for both the size check and the launch
      cap = kda::ring_cap();
      const size_t need = kda::prefill_plan(slot, static_cast<long>(B) * H,
                                            static_cast<int>(nchunk), d_k, d_v, cap)
                              .total;
      if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
        return KDA_ERR_WORKSPACE;
    }
    if (T == 0 && S_T == nullptr) return KDA_OK;

    kda::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
    a.S0 = S0; a.o = o; a.S_T = S_T;
    a.B = B; a.T = T; a.H = H; a.d_k = d_k; a.d_v = d_v; a.chunk = chunk;
    a.gate = gate; a.rule = rule;
    a.fused = fused; a.gate_scale = gate_scale;
    a.bf16 = dtype == KDA_BF16;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    a.ring_cap = cap;
    a.stream = static_cast<hipStream_t>(stream);
    return kda::checked_finish(a.stream, from_hip(noalloc ? kda::launch_prefill_noalloc(a)
                                                           : kda::launch_prefill(a)));
  } catch (...) {
    return KDA_ERR_HIP;
  }
}

int decode_impl(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                float* S, void* o, int B, int H, int d_k, int d_v, int dtype, int gate, int rule,
                bool fused, float gate_scale, void* stream) {
  try {
    if (B < 1 || H < 1 || !dtype_ok(dtype) || !gate_ok(gate) || !rule_ok(rule) ||
        !scale_ok(gate_scale))
      return KDA_ERR_INVALID_ARG;
    if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !beta || !S || !o || (gate != KDA_GATE_NONE && !alpha))
      return KDA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S) || !aligned16(o))
      return KDA_ERR_INVALID_ARG;
    const uintptr_t esz = dtype == KDA_BF16 ? 2 : 4;
    if (gate == KDA_GATE_CHANNEL && !aligned16(alpha)) return KDA_ERR_INVALID_ARG;
    if (gate == KDA_GATE_HEAD && reinterpret_cast<uintptr_t>(alpha) % esz != 0)
      return KDA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(beta) % esz != 0) return KDA_ERR_INVALID_ARG;
    if (static_cast<long long>(B) * H > (1LL << 31) - 1) return KDA_ERR_INVALID_ARG;

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
    a.S = S; a.o = o;
    a.B = B; a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.gate = gate; a.rule = rule;
    a.fused = fused; a.gate_scale = gate_scale;
    a.bf16 = dtype == KDA_BF16;
    a.stream = static_cast<hipStream_t>(stream);
    return kda::checked_finish(a.stream, from_hip(kda::launch_decode(a)));
  } catch (...) {
    return KDA_ERR_HIP;
  }
}

}  // namespace

extern "C" {

int kda_fwd_chunked_ex(const void* q, const void* k, const void* v, const void* alpha,
                       const void* beta, const float* S0, void* o, float* S_T, int B, int T,
                       int H, int d_k, int d_v, int chunk, int dtype, int gate, int rule,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, alpha, beta, S0, o, S_T, B, T, H, d_k, d_v, chunk, dtype, gate, rule,
                  false, 0.f, workspace, workspace_bytes, stream);
}

int kda_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                            const void* beta, const float* S0, void* o, float* S_T, int B, int T,
                            int H, int d_k, int d_v, int chunk, int dtype, int gate, int rule,
                            void* stream) {
  return fwd_impl(q, k, v, alpha, beta, S0, o, S_T, B, T, H, d_k, d_v, chunk, dtype, gate, rule,
                  false, 0.f, nullptr, 0, stream, true);
}

int kda_fwd_chunked(const void* q, const void* k, const void* v, const void* alpha,
                    const void* beta, const float* S0, void* o, float* S_T, int B, int T, int H,
                    int d_k, int d_v, int chunk, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, alpha, beta, S0, o, S_T, B, T, H, d_k, d_v, chunk, dtype,
                  KDA_GATE_CHANNEL, KDA_RULE_DELTA, false, 0.f, workspace, workspace_bytes, stream);
}

int kda_fwd_chunked_fused(const void* q_raw, const void* k_raw, const void* v, const void* g_raw,
                          const void* b_raw, float gate_scale, const float* S0, void* o,
                          float* S_T, int B, int T, int H, int d_k, int d_v, int chunk,
                          int dtype, int gate, int rule, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return fwd_impl(q_raw, k_raw, v, g_raw, b_raw, S0, o, S_T, B, T, H, d_k, d_v, chunk, dtype,
                  gate, rule, true, gate_scale, workspace, workspace_bytes, stream);
}

int kda_decode_step_ex(const void* q, const void* k, const void* v, const void* alpha,
                       const void* beta, float* S, void* o, int B, int H, int d_k, int d_v,
                       int dtype, int gate, int rule, void* stream) {
  return decode_impl(q, k, v, alpha, beta, S, o, B, H, d_k, d_v, dtype, gate, rule, false, 0.f,
                     stream);
}

int kda_decode_step_fused(const void* q_raw, const void* k_raw, const void* v, const void* g_raw,
                          const void* b_raw, float gate_scale, float* S, void* o, int B, int H,
                          int d_k, int d_v, int dtype, int gate, int rule, void* stream) {
  return decode_impl(q_raw, k_raw, v, g_raw, b_raw, S, o, B, H, d_k, d_v, dtype, gate, rule, true,
                     gate_scale, stream);
}

int kda_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                    const void* beta, float* S, void* o, int B, int H, int d_k, int d_v,
                    int dtype, void* stream) {
  return decode_impl(q, k, v, alpha, beta, S, o, B, H, d_k, d_v, dtype, KDA_GATE_CHANNEL,
                     KDA_RULE_DELTA, false, 0.f, stream);
}

}  // extern "C"
