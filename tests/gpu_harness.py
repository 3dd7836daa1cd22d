"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path
through the C ABI binding, and compare against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import gated_delta_rule_76_amd as kda
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(x, y) -> float:
    """max|x - y| / max|y| over the whole tensor (y is the oracle)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.max(np.abs(y))
    return float(np.max(np.abs(x - y)) / (den if den > 0 else 1.0))


def to_dev(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def to_np(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_prefill(x: dict, dtype: str, chunk: int, *, S0=True, alias=False):
    """Upload x (synth arrays) and run kda_fwd_chunked; returns (o, S_T) as fp64 numpy."""
    import torch
    q, k, v, al, be = (to_dev(x[n], dtype) for n in ("q", "k", "v", "alpha", "beta"))
    s0 = None
    if S0 and x.get("S0") is not None:
        s0 = torch.from_numpy(np.ascontiguousarray(x["S0"], dtype=np.float32)).cuda()
    if alias and s0 is not None:
        o, st = kda.kda_fwd_chunked(q, k, v, al, be, s0, chunk=chunk, S_T=s0)
    else:
        o, st = kda.kda_fwd_chunked(q, k, v, al, be, s0, chunk=chunk)
    torch.cuda.synchronize()
    return to_np(o), to_np(st)


def oracle_prefill(x: dict, S0=True, chains=None):
    """Oracle on all chains, or on a list of (b, h) chains; returns o, S_T for those."""
    s0 = x.get("S0") if S0 else None
    if chains is None:
        return oracle.kda_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], s0)
    os_, ss = [], []
    for b, h in chains:
        sl = lambda a: a[b:b + 1, :, h:h + 1]
        o, st = oracle.kda_forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["alpha"]),
                                   sl(x["beta"]), None if s0 is None else s0[b:b + 1, h:h + 1])
        os_.append(o[0, :, 0]); ss.append(st[0, 0])
    return os_, ss
