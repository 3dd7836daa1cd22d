// Host-side interface between the C ABI (kda_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

// Gate kinds and update rules, numbered as kda_gate / kda_rule in kda.h.
constexpr int kGateChannel = 0, kGateHead = 1, kGateNone = 2;
constexpr int kRuleDelta = 0, kRuleLinear = 1;

struct DecodeArgs {
  const void *q, *k, *v, *alpha, *beta;
  float* S;
  void* o;
  int B, H, d_k, d_v;
  int gate, rule;
  bool fused;        // inputs are raw projections: normalise q, k; map the gate and beta
  float gate_scale;  // alpha = exp(-gate_scale * softplus(g)) when fused
  bool bf16;
  hipStream_t stream;
};

struct PrefillArgs {
  const void *q, *k, *v, *alpha, *beta;
  const float* S0;
  void* o;
  float* S_T;
  int B, T, H, d_k, d_v, chunk;
  int gate, rule;
  bool fused;        // inputs are raw projections: normalise q, k; map the gate and beta
  float gate_scale;  // alpha = exp(-gate_scale * softplus(g)) when fused
  bool bf16;
  void* workspace;  // kda_fwd_chunked_workspace_bytes() bytes of device memory
  hipStream_t stream;
};

// Launch one decode step (validated arguments).
hipError_t launch_decode(const DecodeArgs& a);

// Launch the chunked prefill (validated arguments).  Returns
// hipErrorNotSupported when no kernel is compiled for the size combination.
hipError_t launch_prefill(const PrefillArgs& a);

// Whether a prefill kernel exists for this combination (host-only check).
bool prefill_supported(bool bf16, int d_k, int d_v, int chunk);

// Bytes of one chunk's workspace slot for this combination (false when the
// combination is not compiled).  The prefill needs one slot per chunk of
// every (batch, head): B * H * ceil(T / chunk) * slot bytes.
bool prefill_slot_bytes(bool bf16, int d_k, int d_v, int chunk, size_t* slot);

}  // namespace kda
