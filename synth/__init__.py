"""Seeded synthetic inputs for the KDA forward pass.

This module only draws numbers and shapes them; it holds none of the
recurrence's arithmetic.  Both sides of every parity check (the GPU library
and the CPU oracle) take their inputs from here.

Per token and head the method consumes a query q_t, key k_t (length d_k), a
value v_t (length d_v), a per-channel forget gate alpha_t in [0,1]^{d_k} and a
scalar write strength beta_t ("Yanjiu KimiK3 ..." page, sections 3 and 4, the
delta-rule and KDA update equations).  The pages print no workload, so the
distributions below are synthetic stand-ins:

* q, k ~ N(0,1), then L2-normalised per (token, head) over d_k;
* v ~ N(0,1);
* beta = sigmoid(N(0,1));
* alpha = exp(-softplus(N(0,1)) * c) per channel (c = 0.1 or 0.05);
* S0 ~ 0.01 * N(0,1) in fp32 (or zero).

Everything is drawn in float32 from numpy's PCG64 (seeded), normalised in
float32, and, for bf16 workloads, rounded once to bf16 (round to nearest even)
while still stored as float32.  A float32 array that holds bf16-exact values
converts to bf16 on the device without further rounding and to fp64 in the
oracle exactly, so both sides see bit-identical inputs.

Layouts (row-major, contiguous):
    q, k, alpha : [B, T, H, d_k]
    v           : [B, T, H, d_v]
    beta        : [B, T, H]
    S0          : [B, H, d_k, d_v]   (fp32)
Decode steps use T = 1 with the T axis dropped: q [B, H, d_k] and so on.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "round_to_bf16",
    "prefill_inputs",
    "decode_pool",
    "orthonormal_key_set",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32.

    bf16 keeps the top 16 bits of the IEEE-754 float32 pattern.  Adding
    0x7FFF plus the lowest kept bit before truncating rounds to nearest with
    ties to even.  NaN stays NaN (quiet bit forced).
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    r = r.astype(np.uint32)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = (a.view(np.uint32)[nan] | 0x00400000) & 0xFFFF0000
    return r.view(np.float32).reshape(a.shape)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic KDA workload (sizes, gate constant, dtype)."""

    name: str
    B: int
    H: int
    T: int
    d_k: int
    d_v: int
    chunk: int
    dtype: str  # "f32" or "bf16" for q, k, v, alpha, beta and o
    gate_c: float
    s0_std: float  # 0 means S0 = 0
    seed: int
    decode_steps: int = 0  # >0: a decode workload of this many T=1 steps
    notes: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads the build is measured and checked on.  Sizes follow the
# long-context prefill and batched-decode regimes the pages discuss
# (128K-class contexts; a fixed-size state per head replacing the KV cache).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32", 1, 1, 64, 16, 16, 16, "f32", 0.1, 0.0, 0,
                 notes="B1 H1 T64 d16 C16, fp32 end to end"),
        Workload("prefill_h8_t4k", 1, 8, 4096, 128, 128, 64, "bf16", 0.1, 0.01, 1,
                 notes="B1 H8 T4096 d128 C64, bf16 inputs, fp32 state"),
        Workload("prefill_b4_h16_t16k", 4, 16, 16384, 128, 128, 64, "bf16", 0.05, 0.01, 2,
                 notes="B4 H16 T16384 d128 C64"),
        Workload("prefill_h16_t128k", 1, 16, 131072, 128, 128, 64, "bf16", 0.05, 0.01, 3,
                 notes="B1 H16 T131072 d128 C64, 2048 chunks per head"),
        Workload("decode_b256_h16", 256, 16, 1, 128, 128, 0, "bf16", 0.05, 0.01, 4,
                 decode_steps=1000, notes="batched T=1 decode, 1000 steps"),
    ]
}


def _draw_token_tensors(rng: np.random.Generator, lead: tuple, d_k: int, d_v: int,
                        gate_c: float, bf16: bool):
    q = _l2_normalise(rng.standard_normal(lead + (d_k,), dtype=np.float32))
    k = _l2_normalise(rng.standard_normal(lead + (d_k,), dtype=np.float32))
    v = rng.standard_normal(lead + (d_v,), dtype=np.float32)
    xa = rng.standard_normal(lead + (d_k,), dtype=np.float32)
    alpha = np.exp(-_softplus(xa) * np.float32(gate_c)).astype(np.float32)
    del xa
    beta = _sigmoid(rng.standard_normal(lead, dtype=np.float32))
    out = dict(q=q, k=k, v=v, alpha=alpha, beta=beta)
    if bf16:
        out = {n: round_to_bf16(a) for n, a in out.items()}
    return out


def prefill_inputs(B: int, T: int, H: int, d_k: int, d_v: int, *, dtype: str = "bf16",
                   gate_c: float = 0.05, s0_std: float = 0.01, seed: int = 0) -> dict:
    """Draw one prefill batch.  Returns float32 numpy arrays (bf16-exact when
    dtype == "bf16"): q, k, alpha [B,T,H,d_k]; v [B,T,H,d_v]; beta [B,T,H];
    S0 [B,H,d_k,d_v] (None when s0_std == 0)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    out = _draw_token_tensors(rng, (B, T, H), d_k, d_v, gate_c, dtype == "bf16")
    if s0_std > 0:
        out["S0"] = (rng.standard_normal((B, H, d_k, d_v), dtype=np.float32)
                     * np.float32(s0_std)).astype(np.float32)
    else:
        out["S0"] = None
    return out


def workload_inputs(w: Workload, *, T: Optional[int] = None, B: Optional[int] = None,
                    H: Optional[int] = None) -> dict:
    """Inputs of a prefill workload, optionally with a shorter T / B / H."""
    return prefill_inputs(B or w.B, T if T is not None else w.T, H or w.H, w.d_k, w.d_v,
                          dtype=w.dtype, gate_c=w.gate_c, s0_std=w.s0_std, seed=w.seed)


def decode_pool(B: int, H: int, d_k: int, d_v: int, *, pool: int, dtype: str = "bf16",
                gate_c: float = 0.05, s0_std: float = 0.01, seed: int = 4) -> dict:
    """Inputs for batched T=1 decode.

    Returns per-step tensors stacked over a pool of `pool` distinct steps:
    q, k, alpha [pool,B,H,d_k]; v [pool,B,H,d_v]; beta [pool,B,H]; plus the
    initial state S [B,H,d_k,d_v] fp32.  A run of N steps uses pool entry
    (step mod pool) at step `step`.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = _draw_token_tensors(rng, (pool, B, H), d_k, d_v, gate_c, dtype == "bf16")
    out["S"] = (rng.standard_normal((B, H, d_k, d_v), dtype=np.float32)
                * np.float32(s0_std)).astype(np.float32)
    return out


def orthonormal_key_set(d: int, kind: str = "hadamard") -> np.ndarray:
    """d orthonormal keys (rows) whose entries are exact in bf16.

    kind="onehot": the identity; kind="hadamard": a Sylvester Hadamard matrix
    scaled by 1/sqrt(d) (d a power of 4 keeps 1/sqrt(d) a power of two);
    kind="signed": one-hot rows with alternating signs.
    """
    if kind == "onehot":
        return np.eye(d, dtype=np.float32)
    if kind == "signed":
        return np.diag(np.where(np.arange(d) % 2 == 0, 1.0, -1.0)).astype(np.float32)
    if kind == "hadamard":
        h = np.array([[1.0]])
        while h.shape[0] < d:
            h = np.block([[h, h], [h, -h]])
        if h.shape[0] != d:
            raise ValueError("hadamard keys need d a power of two")
        s = 1.0 / np.sqrt(d)
        out = (h * s).astype(np.float32)
        if not np.array_equal(round_to_bf16(out), out):
            raise ValueError("1/sqrt(d) is not exact in bf16 for this d")
        return out
    raise ValueError(kind)
