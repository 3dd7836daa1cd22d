"""fp64 numpy model of the chunked (WY) evaluation the GPU kernels implement.

This is NOT the oracle.  It is a debug-only design model: it spells out the
per-chunk algebra in plain numpy so tests can show that chunking reproduces
the token recurrence exactly (up to rounding) for any chunk size, and so the
kernels' intermediate tiles have a readable reference.

Chunking follows the "Yanjiu KimiK3 ..." page (http://www.pwwt.cn/news/3763336/),
section 6: the sequence is cut into chunks [1,C], [C+1,2C], ...; the state is
passed between chunks and the work inside a chunk is batched into matrix
products, with the chunk's product of rank-one transitions held in the
compact "diagonal minus low rank" form P = D - K W^T of section 6.2.

Per chunk, with rows r = 1..C, gamma_r = prod_{s<=r} alpha_s (per channel):
    K+ = K * gamma          Q+ = Q * gamma         K- = K / gamma
    Kbar = K * gamma_C / gamma
    A = strict_tril(K+ K-^T)        P = tril(Q+ K-^T)
    T = (I + Diag(beta) A)^{-1} Diag(beta)
    U = T (V - K+ S_in)
    O = Q+ S_in + P U
    S_out = Diag(gamma_C) S_in + Kbar^T U
and the chunk's transition product A_C ... A_1 equals Diag(gamma_C) - Kbar^T W
with W = T K+ (the page's D - K W^T).
"""
from __future__ import annotations

import numpy as np


def chunk_tiles(q, k, v, alpha, beta, C: int):
    """Yield per-chunk padded tiles (Q, K, V, alpha, beta, valid) for one chain.

    q, k, alpha: [T, d_k]; v: [T, d_v]; beta: [T].  A short last chunk is
    padded with alpha = 1, beta = 0, k = q = v = 0, which leaves S unchanged.
    """
    T = q.shape[0]
    for t0 in range(0, T, C):
        n = min(C, T - t0)
        Q = np.zeros((C, q.shape[1])); K = np.zeros_like(Q); A = np.ones_like(Q)
        V = np.zeros((C, v.shape[1])); Bt = np.zeros(C)
        Q[:n] = q[t0:t0 + n]; K[:n] = k[t0:t0 + n]; A[:n] = alpha[t0:t0 + n]
        V[:n] = v[t0:t0 + n]; Bt[:n] = beta[t0:t0 + n]
        yield t0, n, Q, K, V, A, Bt


def chunk_factors(K, A, Bt, Q):
    """The S-independent per-chunk factors."""
    C = K.shape[0]
    g = np.cumprod(A, axis=0)
    gC = g[-1]
    Kp = K * g
    Km = K / g
    Qp = Q * g
    Kbar = K * (gC / g)
    Ag = np.tril(Kp @ Km.T, -1)
    P = np.tril(Qp @ Km.T, 0)
    L = np.eye(C) + Bt[:, None] * Ag
    Tm = np.linalg.solve(L, np.diag(Bt))
    return dict(gamma=g, gamma_C=gC, Kp=Kp, Km=Km, Qp=Qp, Kbar=Kbar, A=Ag, P=P, T=Tm, W=Tm @ Kp)


def chunked_forward(q, k, v, alpha, beta, S0=None, C: int = 64):
    """Chunked evaluation, same layouts as the oracle; returns (o, S_T) in fp64."""
    q, k, v, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for t0, n, Q, K, V, Al, Bt in chunk_tiles(q[b, :, h], k[b, :, h], v[b, :, h],
                                                      alpha[b, :, h], beta[b, :, h], C):
                f = chunk_factors(K, Al, Bt, Q)
                U = f["T"] @ (V - f["Kp"] @ S)
                O = f["Qp"] @ S + f["P"] @ U
                S = f["gamma_C"][:, None] * S + f["Kbar"].T @ U
                o[b, t0:t0 + n, h] = O[:n]
            ST[b, h] = S
    return o, ST
