/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * The operation (page "Yanjiu KimiK3, wo faxian damoxing zhengzai xuehui
 * guanli ziji de jisuan", http://www.pwwt.cn/news/3763336/):
 *
 *   state        S_t in R^{d_k x d_v} per (batch, head)            (section 2.1)
 *   update       S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 *                      + beta_t k_t v_t^T,  alpha_t in [0,1]^{d_k}  (section 4)
 *   readout      o_t = S_t^T q_t, taken after the update           (section 2.1)
 *
 * No query scaling and no key normalisation happen inside the library: q and
 * k are used as given.  beta_t is one scalar per (token, head).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates or frees device memory and keeps no state
 *     between calls beyond process-wide caches and settings: the device's
 *     CU count (read once), per kernel whether it has already opted in to
 *     more than 64 KiB of LDS on a device (set once, thread-safely), the
 *     device address of kda_fwd_chunked_noalloc's array (looked up once per
 *     device), the test settings of kda_testing.h, and in the checked build
 *     the site mask of the last failed call.
 *   - Tensors are contiguous and row-major.  Pointers must be 16-byte aligned.
 *   - `dtype` selects the element type of q, k, v, alpha, beta and o:
 *     KDA_F32 (IEEE fp32) or KDA_BF16 (bfloat16).  The state is always fp32.
 *     KDA_F32 computes in fp32 end to end; KDA_BF16 feeds bf16 operands to
 *     the matrix cores with fp32 accumulation and an fp32 state.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.  Argument errors are
 *     reported synchronously, before anything is launched; faults inside a
 *     kernel surface when the caller synchronises the stream.
 *   - Every call returns a kda_status (0 = success).  No C++ exception ever
 *     crosses this boundary.
 *   - Results are deterministic: the same inputs, sizes and stream give
 *     bitwise identical outputs (fixed reduction orders; no atomic ever
 *     accumulates a value).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>

#if defined(__GNUC__) || defined(__clang__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, negative size, misalignment, bad dtype */
    KDA_ERR_UNSUPPORTED = 2, /* valid but not compiled: d_k, d_v, chunk combination */
    KDA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    KDA_ERR_HIP = 4,         /* the HIP runtime rejected a launch */
    KDA_ERR_CHECK = 5        /* checked build only: a kernel index left its buffer (below) */
} kda_status;

/*
 * Gate and update-rule variants, for the *_ex entry points.
 *
 *   KDA_GATE_CHANNEL  alpha holds one decay per key channel, [.., d_k]: the
 *                     KDA gate (section 4, vector gate alpha_t in [0,1]^{d_k}).
 *   KDA_GATE_HEAD     alpha holds one scalar per (token, head), [..] like
 *                     beta: the Gated DeltaNet forget gate that section 4
 *                     starts from, S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
 *                     + beta_t k_t v_t^T (a scalar commutes with the erase).
 *   KDA_GATE_NONE     no decay (alpha = 1); the alpha pointer is not read and
 *                     may be NULL.  With KDA_RULE_DELTA this is the plain
 *                     delta rule of section 3.
 *
 *   KDA_RULE_DELTA    the error-correcting write: the erase term
 *                     -beta_t k_t k_t^T acts on the decayed state (section 3).
 *   KDA_RULE_LINEAR   no correction: S_t = Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *                     the plain additive linear memory of section 2.1 (with
 *                     KDA_GATE_NONE and beta = 1 exactly S_t = S_{t-1} + k_t v_t^T).
 */
typedef enum { KDA_GATE_CHANNEL = 0, KDA_GATE_HEAD = 1, KDA_GATE_NONE = 2 } kda_gate;
typedef enum { KDA_RULE_DELTA = 0, KDA_RULE_LINEAR = 1 } kda_rule;

/* Library ABI version; bumped on any incompatible change. */
KDA_API int kda_version(void);

/* Human-readable name of a kda_status value (static storage, never NULL). */
KDA_API const char *kda_status_string(int status);

/*
 * Checked build.  libkda_checked.so is built from the same sources as
 * libkda.so with bounds checks in every kernel: each index into a global
 * buffer (inputs, outputs, states, the workspace) and each run-time LDS
 * destination of a direct global-to-LDS load is compared with the extent of
 * its buffer before the access.  An index outside it skips the access (a load
 * reads element 0 of the same buffer instead, a store is dropped) and sets
 * the bit of its check site.  Every entry point of the checked build then
 * synchronises its stream and, if any site failed, returns KDA_ERR_CHECK;
 * the outputs of that call are then unspecified.  It is a debugging build:
 * calls are synchronous and slower, and results are otherwise those of
 * libkda.so.  The normal build never returns KDA_ERR_CHECK.
 *
 * kda_build_checked returns 1 in the checked build, 0 in the normal one.
 * kda_check_sites returns the site mask of the last call that returned
 * KDA_ERR_CHECK in the process (0 if none): bits 0-15 prefill kernels
 * (0 q/k rows, 1 gate, 2 beta, 3 workspace slot stores, 4 slot copies,
 * 5 value rows, 6 output rows, 7 S0, 8 S_T, 9 LDS destinations, 10 slot
 * prefetch, 11 self-test), bits 16-23 decode (16 state, 17 q/k/gate, 18 v,
 * 19 beta, 20 output), bits 24-31 AttnRes (24 q, 25 k, 26 h, 27 out).
 */
KDA_API int kda_build_checked(void);
KDA_API unsigned int kda_check_sites(void);

/*
 * kda_fwd_chunked -- prefill: run the recurrence over T tokens for every
 * (batch, head) chain, chunk by chunk.
 *
 * The sequence is cut into chunks of `chunk` tokens; the state is passed from
 * chunk to chunk and each chunk's tokens are processed together through the
 * compact "diagonal minus low rank" form of the chunk's transition product
 * (section 6, chunking and the WY representation P = D - K W^T).  In exact
 * arithmetic the result equals the token-by-token recurrence above.
 *
 *   q, k, alpha : [B, T, H, d_k]   dtype
 *   v           : [B, T, H, d_v]   dtype
 *   beta        : [B, T, H]        dtype
 *   S0          : [B, H, d_k, d_v] fp32, or NULL for a zero initial state
 *   o           : [B, T, H, d_v]   dtype, written (must not alias an input)
 *   S_T         : [B, H, d_k, d_v] fp32, the state after token T-1, or NULL
 *                 to skip it.  S_T may alias S0 (in-place update).
 *   d_k, d_v    : each one of 16, 32, 64, 128
 *   chunk       : one of 16, 32, 64 (KDA_F32 with d_k = 128 supports chunk
 *                 <= 32: its fp32 chunk tiles would not fit in LDS)
 *   workspace   : device memory of at least kda_fwd_chunked_workspace_bytes()
 *                 bytes, 16-byte aligned, owned by the caller.  It holds the
 *                 per-chunk operand tiles between the two kernels of the call
 *                 (a ring of segments for long sequences, see the size query
 *                 below).  Its contents on entry are ignored and undefined on
 *                 return; calls that share a workspace must not overlap in
 *                 time.  NULL or too small -> KDA_ERR_WORKSPACE.
 *
 * Semantics: T = 0 copies S0 (or zeros) to S_T and leaves o untouched.  A
 * last chunk shorter than `chunk` is handled exactly (padding tokens write
 * nothing and do not decay the state).  A NaN or Inf in a chain's inputs at
 * token t makes that chain's outputs from t on and its S_T non-finite;
 * outputs of t's chunk before t may be non-finite too (the chunk's tokens
 * are combined in matrix products), earlier chunks and other chains are
 * unaffected.  In decode a non-finite input stays in its (batch, head).
 * Range of the chunked form: 0 < alpha <= 1 and, per channel, the product
 * of alpha over the tokens of any chunk at least 2^-126 (about e^-87.3; the
 * chunk's decay factors are fp32).  A chunk outside that range (an alpha of
 * exactly 0, or decays that strong) is detected: its chain's outputs from the
 * start of that chunk on and its S_T come out NaN, and the other chains are
 * unaffected.  A smaller chunk widens the range per token (chunk 16 allows
 * four times the per-token decay of chunk 64).  alpha > 1 gives unspecified
 * results.  The decode call below has no such restriction (exact for alpha =
 * 0).
 */
KDA_API int kda_fwd_chunked(const void *q, const void *k, const void *v, const void *alpha,
                    const void *beta, const float *S0, void *o, float *S_T,
                    int B, int T, int H, int d_k, int d_v, int chunk, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_fwd_chunked_ex -- kda_fwd_chunked with a gate and an update rule.
 * Arguments as for kda_fwd_chunked, plus:
 *   gate : kda_gate.  KDA_GATE_HEAD takes alpha as [B, T, H] (dtype);
 *          KDA_GATE_NONE ignores alpha.
 *   rule : kda_rule.
 * kda_fwd_chunked(...) is kda_fwd_chunked_ex(..., KDA_GATE_CHANNEL,
 * KDA_RULE_DELTA, ...).  The workspace size does not depend on gate or rule.
 * A gate or rule outside the enums -> KDA_ERR_INVALID_ARG.
 */
KDA_API int kda_fwd_chunked_ex(const void *q, const void *k, const void *v, const void *alpha,
                       const void *beta, const float *S0, void *o, float *S_T,
                       int B, int T, int H, int d_k, int d_v, int chunk, int dtype,
                       int gate, int rule, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * kda_fwd_chunked_fused -- kda_fwd_chunked_ex from raw projections, with the
 * input maps applied inside the kernels in fp32 (the step before the
 * recurrence: unit keys for the projection reading of section 3, a gate in
 * [0, 1] per section 4):
 *   q_raw, k_raw : [B, T, H, d_k] dtype; the library uses q = q_raw / |q_raw|
 *                  and k = k_raw / |k_raw| per (token, head) (a zero vector
 *                  stays zero)
 *   g_raw        : gate projection, [B, T, H, d_k] (KDA_GATE_CHANNEL) or
 *                  [B, T, H] (KDA_GATE_HEAD), dtype; alpha = exp(-gate_scale *
 *                  softplus(g_raw)), softplus(x) = log(1 + e^x).  Ignored
 *                  (may be NULL) with KDA_GATE_NONE.
 *   b_raw        : [B, T, H] dtype; beta = sigmoid(b_raw) = 1 / (1 + e^-b_raw)
 *   gate_scale   : c >= 0, finite; otherwise KDA_ERR_INVALID_ARG
 * v is used as given.  All other arguments, the workspace and the semantics
 * are those of kda_fwd_chunked_ex.  Safe range of the raw gate (the range
 * of the chunked form above): per channel, c * sum softplus(g_raw) over the
 * tokens of any chunk at most 87; on average c * softplus(g_raw) <= 1.36 at
 * chunk 64, <= 2.7 at chunk 32, <= 5.4 at chunk 16 (softplus(0) = 0.69).
 * Chunks beyond it give NaN as described for kda_fwd_chunked.
 */
KDA_API int kda_fwd_chunked_fused(const void *q_raw, const void *k_raw, const void *v,
                          const void *g_raw, const void *b_raw, float gate_scale,
                          const float *S0, void *o, float *S_T, int B, int T, int H, int d_k,
                          int d_v, int chunk, int dtype, int gate, int rule, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * kda_fwd_chunked_noalloc -- kda_fwd_chunked_ex with no workspace argument,
 * for callers that cannot allocate device memory (code under stream or graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments
 * and results are those of kda_fwd_chunked_ex; the operand slots live in a
 * device array inside the library instead of a caller workspace.
 *
 * The array is 64 MiB per GPU (held from the library's load until the
 * process ends) and is shared by every call on that GPU: calls that overlap
 * in time on one GPU (on different streams or from different threads) race
 * and give undefined results.  Nothing in it needs clearing between calls.
 * The sequence runs in as many segments as the array needs (slower than
 * kda_fwd_chunked with a full-size workspace for long sequences).  Sizes for
 * which one chunk of every (batch, head) chain per ring buffer plus the
 * carried states do not fit the array (B * H above about 350 at d = 128,
 * chunk = 64, bf16, once the slots of the whole call exceed 64 MiB) return
 * KDA_ERR_WORKSPACE before anything is launched.  No hipMalloc, hipFree or
 * allocating library routine is called.
 */
KDA_API int kda_fwd_chunked_noalloc(const void *q, const void *k, const void *v,
                            const void *alpha, const void *beta, const float *S0, void *o,
                            float *S_T, int B, int T, int H, int d_k, int d_v, int chunk,
                            int dtype, int gate, int rule, void *stream);

/* Bytes of workspace kda_fwd_chunked needs for these sizes.  It holds one
 * operand slot (61 KiB at d_k = d_v = 128, chunk = 64, bf16) per (chain,
 * chunk) while they fit 512 MiB: B * H * ceil(T / chunk) slots.  Beyond that
 * the sequence runs in segments through two ring buffers of at least one
 * chunk of every chain each, plus one carried fp32 state per chain, so the
 * size stops growing with T.  0 for an unsupported or invalid combination. */
KDA_API size_t kda_fwd_chunked_workspace_bytes(int B, int T, int H, int d_k, int d_v,
                                       int chunk, int dtype);

/*
 * kda_decode_step -- one token per sequence (T = 1), state updated in place.
 *
 * Per (b, h): S' = Diag(alpha) S; v_hat = S'^T k (the delta rule's
 * prediction, section 3); u = beta (v - v_hat); S <- S' + k u^T; and
 * o = S^T q, computed as S'^T q + (k^T q) u in the same single pass over S.
 *
 *   q, k, alpha : [B, H, d_k]      dtype
 *   v           : [B, H, d_v]      dtype
 *   beta        : [B, H]           dtype
 *   S           : [B, H, d_k, d_v] fp32, read and overwritten in place
 *   o           : [B, H, d_v]      dtype, written
 *   d_k, d_v    : each one of 16, 32, 64, 128
 *
 * Exact for any alpha in [0,1], including alpha = 0.
 */
KDA_API int kda_decode_step(const void *q, const void *k, const void *v, const void *alpha,
                    const void *beta, float *S, void *o, int B, int H, int d_k, int d_v,
                    int dtype, void *stream);

/*
 * kda_decode_step_ex -- kda_decode_step with a gate and an update rule (see
 * kda_gate, kda_rule).  KDA_GATE_HEAD takes alpha as [B, H]; KDA_GATE_NONE
 * ignores alpha.  KDA_RULE_LINEAR drops the prediction: u = beta v.
 */
KDA_API int kda_decode_step_ex(const void *q, const void *k, const void *v, const void *alpha,
                       const void *beta, float *S, void *o, int B, int H, int d_k, int d_v,
                       int dtype, int gate, int rule, void *stream);

/*
 * kda_decode_step_fused -- kda_decode_step_ex from raw projections, with the
 * same input maps as kda_fwd_chunked_fused (q, k L2-normalised; alpha =
 * exp(-gate_scale * softplus(g_raw)); beta = sigmoid(b_raw)).  g_raw is
 * [B, H, d_k] or [B, H] by gate; b_raw is [B, H].
 */
KDA_API int kda_decode_step_fused(const void *q_raw, const void *k_raw, const void *v,
                          const void *g_raw, const void *b_raw, float gate_scale, float *S,
                          void *o, int B, int H, int d_k, int d_v, int dtype, int gate, int rule,
                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
