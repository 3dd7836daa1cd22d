"""fp64 CPU oracle for AttnRes depth aggregation.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the GPU library never does.

Definition (page "Yanjiu KimiK3 ...", http://www.pwwt.cn/news/3763336/,
section 8, the AttnRes equations): a layer l takes the outputs of the layers
before it, h_1 .. h_{l-1}, weighs them with softmax(q_l^T k_i) over i < l
and sums:   h_l = sum_{i<l} alpha_{i->l} h_i,  alpha_{i->l} = softmax_i(q_l^T k_i).
Per token.  The pages give no scale inside the softmax, so there is none.

Layout: q [N, d_k] (the current layer's query per token), k [L, N, d_k] and
h [L, N, d] (key and output of each of the L earlier layers per token).
Returns out [N, d] in fp64.
"""
from __future__ import annotations

import numpy as np


def attnres_forward(q, k, h) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    L, N, dk = k.shape
    if q.shape != (N, dk) or h.shape[:2] != (L, N) or L < 1:
        raise ValueError("q must be [N,d_k], k [L,N,d_k], h [L,N,d], L >= 1")
    scores = np.einsum("nc,lnc->nl", q, k)              # q_l^T k_i for every token
    scores -= scores.max(axis=1, keepdims=True)         # softmax is shift invariant
    w = np.exp(scores)
    w /= w.sum(axis=1, keepdims=True)                   # alpha_{i->l}, rows sum to 1
    return np.einsum("nl,lnd->nd", w, h)
