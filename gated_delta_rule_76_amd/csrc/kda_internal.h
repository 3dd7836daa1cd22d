// Host-side interface between the C ABI (kda_api.hip) and the kernel files.
#pragma once

#include <stddef.h>

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
  void* workspace;         // at least prefill_plan(...).total bytes of device memory
  size_t workspace_bytes;
  size_t ring_cap;         // segment ring budget the plan was made with
  hipStream_t stream;
};

// How a prefill call walks the sequence.  The prep kernel writes one
// operand slot per (chain, chunk) and the state pass reads it back; when all
// slots would take more than `ring_cap` bytes, the chunks are cut into
// segments of `seg` chunks that run one after the other through two ring
// buffers of `half` bytes each, the state passing from one segment to the
// next through S_T or, without S_T, through a carrier area of
// nchain * d_k * d_v fp32 at carrier_off.  The workspace then no longer grows
// with the sequence length.
struct PrefillPlan {
  int seg = 0;             // chunks per segment
  int nseg = 0;            // segments (1 when everything fits)
  int nbuf = 1;            // ring buffers in use (2 when segmented)
  size_t half = 0;         // bytes of one segment's slots (256-byte aligned)
  size_t carrier_off = 0;  // byte offset of the carrier area (segmented only)
  size_t total = 0;        // workspace bytes the call needs
};

constexpr size_t kRingCap = size_t(512) << 20;  // slot budget of kda_fwd_chunked

inline PrefillPlan prefill_plan(size_t slot, long nchain, int nchunk, int d_k, int d_v,
                                size_t cap) {
  PrefillPlan p;
  const size_t full = slot * static_cast<size_t>(nchain) * static_cast<size_t>(nchunk);
  if (full <= cap || nchunk <= 1) {
    p.seg = nchunk;
    p.nseg = 1;
    p.half = full;
    p.total = full;
    return p;
  }
  const size_t per_chunk = slot * static_cast<size_t>(nchain);
  size_t lmax = cap / (2 * per_chunk);
  if (lmax < 1) lmax = 1;
  p.nseg = static_cast<int>((static_cast<size_t>(nchunk) + lmax - 1) / lmax);
  p.seg = (nchunk + p.nseg - 1) / p.nseg;
  p.nbuf = 2;
  p.half = (per_chunk * static_cast<size_t>(p.seg) + 255) / 256 * 256;
  p.carrier_off = 2 * p.half;
  p.total = p.carrier_off + static_cast<size_t>(nchain) * d_k * d_v * sizeof(float);
  return p;
}

// Polls an output wave of the prefill state pass makes while it waits for
// the state wave's U of a chunk before it gives up and writes NaN for that
// chunk (default 1 << 24; kda_testing_set_wait_limit changes it).
int wait_limit();

// Size of the device array behind kda_fwd_chunked_noalloc (per GPU).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

// Ring budget for an allocation-free prefill of these sizes, such that the
// whole plan fits kNoAllocScratchBytes; false when no plan fits (too many
// (batch, head) chains for one chunk of each per ring buffer).
bool noalloc_plan(size_t slot, long nchain, int nchunk, int d_k, int d_v, size_t* cap);

// Launch the chunked prefill in the library's own device array (validated
// arguments; a.ring_cap from noalloc_plan).  Allocates nothing.
hipError_t launch_prefill_noalloc(const PrefillArgs& a);

// Slot budget of kda_fwd_chunked's segment ring (kRingCap unless a test
// changed it with kda_testing_set_ring_cap).
size_t ring_cap();

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

// Checked build (bounds checks in the kernels, see kda_check.h): each unit's
// failed check sites on the current device since its last take (always 0 in
// the normal build).
unsigned prefill_check_take();
unsigned decode_check_take();
unsigned attnres_check_take();
// A kernel whose one check fails on purpose, touching no memory (the checked
// build's self-test; a no-op kernel in the normal build).
hipError_t launch_check_probe(hipStream_t stream);
// End of an entry point: in the checked build, synchronise `stream`, collect
// every unit's failed sites and report any as KDA_ERR_CHECK (the mask is kept
// for kda_check_sites); in the normal build, `status` unchanged.
int checked_finish(hipStream_t stream, int status);

}  // namespace kda
