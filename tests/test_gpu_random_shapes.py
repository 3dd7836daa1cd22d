"""Seeded random sweeps of prefill and decode shapes and variants against the fp64
oracle: element type, key and value widths, chunk size, batch, heads,
sequence length (ragged chunks and T below one chunk included), gate kind,
update rule, with or without an initial state, and the segment-ring budget
(default, or small enough to cut the sequence into several segments); and
three decode steps per drawn decode shape and variant.  The draws are fixed
(seeds 2024 and 4242), so every run checks the same 24 + 16 cases."""
import numpy as np
import pytest

import oracle
from synth import prefill_inputs
from tests.gpu_harness import TOL, log, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < n:
        dtype = ["f32", "bf16"][rng.integers(2)]
        dk = int(rng.choice([16, 32, 64, 128]))
        dv = int(rng.choice([16, 32, 64, 128]))
        C = int(rng.choice([16, 32, 64]))
        if dtype == "f32" and dk == 128 and C == 64:
            continue  # not compiled: the fp32 chunk tiles would not fit in LDS
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        T = int(rng.integers(1, 301))
        gate = ["channel", "head", "none"][rng.integers(3)]
        rule = ["delta", "linear"][rng.integers(2)]
        s0 = bool(rng.integers(2))
        small_ring = bool(rng.integers(2))
        out.append((dtype, dk, dv, C, B, T, H, gate, rule, s0, small_ring))
    return out


@pytest.mark.parametrize("dtype,dk,dv,C,B,T,H,gate,rule,s0,small_ring", _cases())
def test_random_prefill_case(dtype, dk, dv, C, B, T, H, gate, rule, s0, small_ring):
    import torch
    import gated_delta_rule_76_amd as kda
    name = (f"{dtype} dk{dk} dv{dv} C{C} B{B} T{T} H{H} {gate}/{rule} S0={s0} "
            f"ring={'small' if small_ring else 'default'}")
    log(f"[random prefill] {name}")
    x = prefill_inputs(B, T, H, dk, dv, dtype=dtype, gate_c=0.1, s0_std=0.05 if s0 else 0.0,
                       seed=T * 7 + dk + dv + C)
    alpha = {"channel": x["alpha"], "head": np.ascontiguousarray(x["alpha"][..., 0]),
             "none": None}[gate]
    default = kda.ring_cap()
    try:
        if small_ring:
            # room for about three chunks of slots: several segments whenever
            # the sequence has more than one or two chunks
            slot = kda.workspace_bytes(1, C, 1, dk, dv, C, kda.KDA_BF16 if dtype == "bf16" else kda.KDA_F32)
            assert kda.set_ring_cap(max(3 * B * H * slot, 1)) == 0
        q, k, v, be = (to_dev(x[n], dtype) for n in ("q", "k", "v", "beta"))
        al = None if alpha is None else to_dev(alpha, dtype)
        S0 = torch.from_numpy(x["S0"]).cuda() if s0 else None
        o, st = kda.kda_fwd_chunked(q, k, v, al, be, S0, chunk=C, gate=gate, rule=rule)
        torch.cuda.synchronize()
    finally:
        assert kda.set_ring_cap(default) == 0
    o_ref, s_ref = oracle.kda_forward(x["q"], x["k"], x["v"], alpha, x["beta"], x["S0"] if s0 else None,
                                      gate=gate, rule=rule)
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(st), s_ref)
    log(f"  rel_err o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def _decode_cases(n=16, seed=4242):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [(["f32", "bf16"][rng.integers(2)], int(rng.choice([16, 32, 64, 128])),
             int(rng.choice([16, 32, 64, 128])), int(rng.integers(1, 5)), int(rng.integers(1, 6)),
             ["channel", "head", "none"][rng.integers(3)], ["delta", "linear"][rng.integers(2)])
            for _ in range(n)]


@pytest.mark.parametrize("dtype,dk,dv,B,H,gate,rule", _decode_cases())
def test_random_decode_case(dtype, dk, dv, B, H, gate, rule):
    """Three consecutive decode steps on a random shape and variant (seed 4242)."""
    import torch
    import gated_delta_rule_76_amd as kda
    from synth import decode_pool
    log(f"[random decode] {dtype} dk{dk} dv{dv} B{B} H{H} {gate}/{rule}")
    p = decode_pool(B, H, dk, dv, pool=3, dtype=dtype, gate_c=0.1, s0_std=0.05, seed=dk * 3 + dv + B * H)
    S = torch.from_numpy(p["S"]).cuda()
    Sref = p["S"].astype(np.float64)
    for i in range(3):
        a = {"channel": p["alpha"][i], "head": np.ascontiguousarray(p["alpha"][i][..., 0]),
             "none": None}[gate]
        dev = {n: to_dev(p[n][i], dtype) for n in ("q", "k", "v", "beta")}
        o = kda.kda_decode_step(dev["q"], dev["k"], dev["v"], None if a is None else to_dev(a, dtype),
                                dev["beta"], S, gate=gate, rule=rule)
        o_ref, Sref = oracle.kda_decode_step(p["q"][i], p["k"][i], p["v"][i], a, p["beta"][i], Sref,
                                             gate=gate, rule=rule)
        torch.cuda.synchronize()
        assert rel_err(to_np(o), o_ref) <= TOL[dtype], i
    es = rel_err(S.cpu().numpy(), Sref)
    log(f"  rel_err S {es:.2e}")
    assert es <= TOL[dtype]
