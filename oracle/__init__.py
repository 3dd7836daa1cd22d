"""fp64 CPU oracle for the KDA forward pass.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The GPU library never does,
and this package imports nothing from it: the two share no code.

The arithmetic lives in ``kda_oracle.c`` (plain C, OpenMP over independent
(batch, head) chains): a token-by-token fp64 evaluation of the KDA update
S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T with the
readout o_t = S_t^T q_t (page "Yanjiu KimiK3 ...", http://www.pwwt.cn/news/3763336/,
section 4 KDA update equation and section 2.1 read equation).  This module
only marshals numpy arrays into it.

Every function here is pinned by CPU tests against closed forms, special
cases and exact rational arithmetic (see tests/test_oracle_pins.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None

NO_CORRECTION = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                        "-fno-fast-math", "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            d = ctypes.POINTER(ctypes.c_double)
            lib.kda_oracle_fwd.argtypes = [d, d, d, d, d, d, d, d, ctypes.c_long, ctypes.c_long,
                                           ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                           ctypes.c_int, ctypes.c_int]
            lib.kda_oracle_fwd.restype = ctypes.c_int
            lib.kda_oracle_max_threads.argtypes = []
            lib.kda_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _gate_to_channels(alpha, gate: str, shape):
    """The gate as one decay per key channel.  A per-head scalar gate (the
    Gated DeltaNet form alpha_t (I - beta_t k_t k_t^T) S_{t-1}, page "Yanjiu
    KimiK3 ...", section 4) is that scalar on every channel: a scalar
    commutes with the erase, so it is the per-channel recurrence with all
    channels equal.  No gate is alpha = 1."""
    if gate == "channel":
        return _f64(alpha)
    if gate == "head":
        return np.ascontiguousarray(np.broadcast_to(_f64(alpha)[..., None], shape))
    if gate == "none":
        return np.ones(shape, dtype=np.float64)
    raise ValueError(f"unknown gate {gate!r}")


def kda_forward(q, k, v, alpha, beta, S0=None, *, no_correction: bool = False,
                gate: str = "channel", rule: str = "delta",
                threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token fp64 KDA forward.

    q, k: [B,T,H,d_k]; alpha: [B,T,H,d_k] (gate "channel"), [B,T,H] (gate
    "head") or ignored (gate "none"); v: [B,T,H,d_v]; beta: [B,T,H];
    S0: [B,H,d_k,d_v] or None (zero state).  rule "linear" (or
    no_correction=True) drops the prediction: the write is beta_t k_t v_t^T
    (section 2.1's additive memory).  Returns (o [B,T,H,d_v], S_T), fp64.
    """
    if rule not in ("delta", "linear"):
        raise ValueError(f"unknown rule {rule!r}")
    no_correction = no_correction or rule == "linear"
    q, k, v, beta = (_f64(x) for x in (q, k, v, beta))
    if q.ndim != 4:
        raise ValueError("q must be [B,T,H,d_k]")
    alpha = _gate_to_channels(alpha, gate, q.shape)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or alpha.shape != q.shape:
        raise ValueError("k and alpha must have q's shape")
    if v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("v must be [B,T,H,d_v] and beta [B,T,H]")
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None and s0.shape != (B, H, dk, dv):
        raise ValueError("S0 must be [B,H,d_k,d_v]")
    o = np.empty((B, T, H, dv), dtype=np.float64)
    ST = np.empty((B, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0),
                                _ptr(o), _ptr(ST), B, T, H, dk, dv,
                                NO_CORRECTION if no_correction else 0, int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed with code {rc}")
    return o, ST


def kda_decode_step(q, k, v, alpha, beta, S, *, gate: str = "channel", rule: str = "delta",
                    threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """One T=1 step: q, k [B,H,d_k]; alpha [B,H,d_k] / [B,H] / ignored by gate;
    v [B,H,d_v]; beta [B,H]; S [B,H,d_k,d_v].  Returns (o [B,H,d_v], S_new),
    fp64.  Same recurrence as kda_forward."""
    q, k, v = (_f64(x)[:, None] for x in (q, k, v))
    alpha = None if gate == "none" else _f64(alpha)[:, None]
    beta = _f64(beta)[:, None]
    o, ST = kda_forward(q, k, v, alpha, beta, S, gate=gate, rule=rule, threads=threads)
    return o[:, 0], ST


def input_prologue(q_raw, k_raw, g_raw, b_raw, gate_scale: float, gate: str = "channel"):
    """The input maps in front of the recurrence, in fp64 (the fused kernels
    apply them in fp32): unit query and key per (token, head) (the projection
    reading of the delta rule, page "Yanjiu KimiK3 ...", section 3, needs unit
    keys), a gate in [0, 1] (section 4) as alpha = exp(-c softplus(g)), and
    beta = sigmoid(b).  A zero vector stays zero.  Returns (q, k, alpha, beta);
    alpha keeps g_raw's shape (None for gate "none")."""
    def unit(x):
        x = _f64(x)
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)
    q, k = unit(q_raw), unit(k_raw)
    alpha = None
    if gate != "none":
        g = _f64(g_raw)
        softplus = np.maximum(g, 0.0) + np.log1p(np.exp(-np.abs(g)))
        alpha = np.exp(-float(gate_scale) * softplus)
    beta = 1.0 / (1.0 + np.exp(-_f64(b_raw)))
    return q, k, alpha, beta


def kda_forward_fused(q_raw, k_raw, v, g_raw, b_raw, S0=None, *, gate_scale: float,
                      gate: str = "channel", rule: str = "delta", threads: int = 0):
    """kda_forward on the prologue's outputs (fp64 end to end)."""
    q, k, alpha, beta = input_prologue(q_raw, k_raw, g_raw, b_raw, gate_scale, gate)
    return kda_forward(q, k, v, alpha, beta, S0, gate=gate, rule=rule, threads=threads)
