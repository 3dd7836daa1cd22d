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

Everything is drawn in float32 from numpy's PCG64 and normalised in float32;
for bf16 workloads it is then rounded once to bf16 (round to nearest even)
while still stored as float32.  A float32 array that holds bf16-exact values
converts to bf16 on the device without further rounding and to fp64 in the
oracle exactly, so both sides see bit-identical inputs.

Seeding: the flattened (batch, token, head) rows are cut into fixed blocks of
32768 rows; block j of tensor i draws from PCG64(SeedSequence([seed, i, j])).
Blocks are filled by a thread pool, and the bytes do not depend on the
number of threads.

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
    "decode_steps",
    "decode_state",
    "orthonormal_key_set",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32.

    bf16 keeps the top 16 bits of the IEEE-754 float32 pattern.  Adding
    0x7FFF plus the lowest kept bit before truncating rounds to nearest with
    ties to even.  NaN stays NaN (quiet bit forced).
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                      # wraps only for NaN patterns, fixed below
    r &= np.uint32(0xFFFF0000)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = (u[nan] | np.uint32(0x00400000)) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(a.shape)


def _l2_normalise_(x: np.ndarray) -> None:
    n = np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float32))
    x /= np.maximum(n, np.float32(1e-12))[..., None]


# Rows (token-heads) per independently seeded block.  Fixed, so the bytes
# drawn do not depend on how many threads generate them.
_BLOCK = 1 << 15
_TENSORS = ("q", "k", "v", "alpha", "beta")


def _fill_block(out: dict, tid_seed, j: int, d_k: int, d_v: int, gate_c: float,
                bf16: bool, rows: int = _BLOCK) -> None:
    """Fill rows [j*rows, (j+1)*rows) of every token tensor.  `tid_seed` is an
    int or a tuple of ints; block j of tensor i draws from
    PCG64(SeedSequence([*tid_seed, i, j]))."""
    lo = j * rows
    hi = min(lo + rows, out["q"].shape[0])
    n = hi - lo
    prefix = list(tid_seed) if isinstance(tid_seed, tuple) else [tid_seed]
    for ti, name in enumerate(_TENSORS):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(prefix + [ti, j])))
        if name in ("q", "k"):
            x = rng.standard_normal((n, d_k), dtype=np.float32)
            _l2_normalise_(x)
        elif name == "v":
            x = rng.standard_normal((n, d_v), dtype=np.float32)
        elif name == "alpha":
            x = rng.standard_normal((n, d_k), dtype=np.float32)
            np.logaddexp(np.float32(0.0), x, out=x)          # softplus
            x *= np.float32(-gate_c)
            np.exp(x, out=x)                                  # exp(-c softplus)
        else:
            x = rng.standard_normal(n, dtype=np.float32)
            np.negative(x, out=x)
            np.exp(x, out=x)
            x += np.float32(1.0)
            np.reciprocal(x, out=x)                           # sigmoid
        out[name][lo:hi] = round_to_bf16(x) if bf16 else x


def _draw_token_tensors(seed: int, lead: tuple, d_k: int, d_v: int, gate_c: float,
                        bf16: bool) -> dict:
    import concurrent.futures as cf
    import os

    N = int(np.prod(lead)) if lead else 1
    out = {"q": np.empty((N, d_k), np.float32), "k": np.empty((N, d_k), np.float32),
           "v": np.empty((N, d_v), np.float32), "alpha": np.empty((N, d_k), np.float32),
           "beta": np.empty((N,), np.float32)}
    nblk = (N + _BLOCK - 1) // _BLOCK
    workers = max(1, min(nblk, os.cpu_count() or 1, 16))
    if workers == 1:
        for j in range(nblk):
            _fill_block(out, seed, j, d_k, d_v, gate_c, bf16)
    else:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda j: _fill_block(out, seed, j, d_k, d_v, gate_c, bf16), range(nblk)))
    return {n: a.reshape(lead + a.shape[1:]) for n, a in out.items()}


def _draw_state(seed: int, shape: tuple, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    return x


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


def prefill_inputs(B: int, T: int, H: int, d_k: int, d_v: int, *, dtype: str = "bf16",
                   gate_c: float = 0.05, s0_std: float = 0.01, seed: int = 0) -> dict:
    """Draw one prefill batch.  Returns float32 numpy arrays (bf16-exact when
    dtype == "bf16"): q, k, alpha [B,T,H,d_k]; v [B,T,H,d_v]; beta [B,T,H];
    S0 [B,H,d_k,d_v] (None when s0_std == 0)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    out = _draw_token_tensors(seed, (B, T, H), d_k, d_v, gate_c, dtype == "bf16")
    out["S0"] = _draw_state(seed, (B, H, d_k, d_v), s0_std) if s0_std > 0 else None
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
    out = _draw_token_tensors(seed, (pool, B, H), d_k, d_v, gate_c, dtype == "bf16")
    out["S"] = _draw_state(seed, (B, H, d_k, d_v), s0_std)
    return out


# Entropy tag of per-step decode draws (keeps them apart from prefill draws).
_DECODE_TAG = 0xDEC0DE


def decode_state(B: int, H: int, d_k: int, d_v: int, *, s0_std: float = 0.01,
                 seed: int = 4) -> np.ndarray:
    """Initial fp32 state S [B,H,d_k,d_v] = s0_std * N(0,1) of a decode run."""
    return _draw_state(seed, (B, H, d_k, d_v), s0_std)


def decode_steps(B: int, H: int, d_k: int, d_v: int, first: int, count: int, *,
                 dtype: str = "bf16", gate_c: float = 0.05, seed: int = 4) -> dict:
    """Inputs of decode steps first .. first+count-1, stacked on a leading step
    axis: q, k, alpha [count,B,H,d_k]; v [count,B,H,d_v]; beta [count,B,H]
    (float32, bf16-exact when dtype == "bf16").  Step s draws tensor i from
    PCG64(SeedSequence([seed, tag, s, i, 0])), so its values depend on (seed, s)
    alone and a long run can be drawn in pieces; every step is distinct."""
    import concurrent.futures as cf
    import os

    rows = B * H
    out = {"q": np.empty((count * rows, d_k), np.float32),
           "k": np.empty((count * rows, d_k), np.float32),
           "v": np.empty((count * rows, d_v), np.float32),
           "alpha": np.empty((count * rows, d_k), np.float32),
           "beta": np.empty((count * rows,), np.float32)}

    def one(i):
        # each step is its own block of B*H rows; views keep step i's rows apart
        view = {n: a[i * rows:(i + 1) * rows] for n, a in out.items()}
        _fill_block(view, (seed, _DECODE_TAG, first + i), 0, d_k, d_v, gate_c, dtype == "bf16",
                    rows=rows)

    workers = max(1, min(count, os.cpu_count() or 1, 16))
    if workers == 1:
        for i in range(count):
            one(i)
    else:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(count)))
    lead = (count, B, H)
    return {n: a.reshape(lead + a.shape[1:]) for n, a in out.items()}


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


def raw_prefill_inputs(B: int, T: int, H: int, d_k: int, d_v: int, *, dtype: str = "bf16",
                       s0_std: float = 0.01, seed: int = 0) -> dict:
    """Raw projections for the fused prologue: q_raw, k_raw [B,T,H,d_k],
    v [B,T,H,d_v], g_raw [B,T,H,d_k] (a per-head gate takes [..., 0]),
    b_raw [B,T,H], all N(0, 1) draws (bf16-exact when dtype == "bf16"), and
    S0 = s0_std * N(0, 1) fp32.  No maps are applied here."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7777])))
    out = {
        "q_raw": rng.standard_normal((B, T, H, d_k), dtype=np.float32),
        "k_raw": rng.standard_normal((B, T, H, d_k), dtype=np.float32),
        "v": rng.standard_normal((B, T, H, d_v), dtype=np.float32),
        "g_raw": rng.standard_normal((B, T, H, d_k), dtype=np.float32),
        "b_raw": rng.standard_normal((B, T, H), dtype=np.float32),
    }
    if dtype == "bf16":
        out = {n: round_to_bf16(a) for n, a in out.items()}
    out["S0"] = (s0_std * rng.standard_normal((B, H, d_k, d_v))).astype(np.float32) if s0_std > 0 else None
    return out


def attnres_inputs(L: int, N: int, d_k: int, d: int, *, dtype: str = "bf16", seed: int = 0) -> dict:
    """AttnRes inputs: q [N,d_k], k [L,N,d_k] ~ N(0, 1/sqrt(d_k)) each (so a
    score q.k has unit variance), h [L,N,d] ~ N(0,1); float32, bf16-exact when
    dtype == "bf16"."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4242])))
    s = d_k ** -0.25
    out = {"q": (s * rng.standard_normal((N, d_k))).astype(np.float32),
           "k": (s * rng.standard_normal((L, N, d_k))).astype(np.float32),
           "h": rng.standard_normal((L, N, d), dtype=np.float32)}
    if dtype == "bf16":
        out = {n: round_to_bf16(a) for n, a in out.items()}
    return out
