/*
 * attnres.h -- C ABI of the AttnRes depth aggregation kernel (gfx950).
 *
 * The operation (page "Yanjiu KimiK3, wo faxian damoxing zhengzai xuehui
 * guanli ziji de jisuan", http://www.pwwt.cn/news/3763336/, section 8):
 * a layer reads the outputs h_1 .. h_{l-1} of the layers before it, weighs
 * them with alpha_{i->l} = softmax_i(q_l^T k_i) and sums them,
 *   h_l = sum_{i<l} alpha_{i->l} h_i,
 * independently for every token.  No scale is applied inside the softmax.
 *
 * Conventions as in kda.h: device pointers owned by the caller, contiguous
 * row-major tensors, 16-byte aligned; work enqueued on `stream` without
 * synchronising; errors returned synchronously as kda_status values (0 = OK,
 * 1 = invalid argument, 2 = unsupported size, 4 = HIP launch failure);
 * deterministic results.  The library allocates nothing.
 */
#ifndef ATTNRES_H_
#define ATTNRES_H_

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attnres_forward
 *   q    : [N, d_k]     dtype (KDA_F32 or KDA_BF16), the current layer's query
 *   k    : [L, N, d_k]  dtype, the key of each earlier layer
 *   h    : [L, N, d]    dtype, the output of each earlier layer
 *   out  : [N, d]       dtype, written; must not overlap q, k or h
 *   1 <= L <= 1024, 1 <= d_k <= 512, d a positive multiple of 8, N >= 1.
 * Scores and the weighted sum are accumulated in fp32 (max-subtracted
 * softmax); out is rounded to dtype once.
 */
KDA_API int attnres_forward(const void *q, const void *k, const void *h, void *out, int L, int N,
                            int d_k, int d, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H_ */
