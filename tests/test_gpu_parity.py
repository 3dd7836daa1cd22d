"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: max|gpu - oracle| / max|oracle| per tensor (o and S_T separately)
<= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest

import oracle
from synth import WORKLOADS, decode_pool, prefill_inputs, workload_inputs
from tests.gpu_harness import TOL, log, oracle_prefill, rel_err, run_prefill, to_dev, to_np

pytestmark = pytest.mark.gpu


def _check(name, o, st, o_ref, s_ref, tol):
    eo, es = rel_err(o, o_ref), rel_err(st, s_ref)
    log(f"[{name}] rel_err o={eo:.3e} S_T={es:.3e} (tol {tol:g})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(st))
    assert eo <= tol and es <= tol


def _sampled(x, chains):
    """Stack the listed (b, h) chains as heads of one batch for the oracle."""
    sel = lambda a: np.stack([a[b, :, h] for b, h in chains], axis=1)[None]
    s0 = None if x.get("S0") is None else np.stack([x["S0"][b, h] for b, h in chains])[None]
    return oracle.kda_forward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["alpha"]),
                              sel(x["beta"]), s0)


# ------------------------------------------------------------ named workloads
def test_tiny_f32_full():
    w = WORKLOADS["tiny_f32"]
    log(f"[tiny_f32] B{w.B} H{w.H} T{w.T} d{w.d_k} C{w.chunk} f32")
    x = workload_inputs(w)
    o, st = run_prefill(x, "f32", w.chunk)
    o_ref, s_ref = oracle_prefill(x)
    _check("tiny_f32", o, st, o_ref, s_ref, TOL["f32"])


def test_prefill_h8_t4k_full():
    w = WORKLOADS["prefill_h8_t4k"]
    log(f"[prefill_h8_t4k] B{w.B} H{w.H} T{w.T} d{w.d_k} C{w.chunk} bf16")
    x = workload_inputs(w)
    o, st = run_prefill(x, "bf16", w.chunk)
    o_ref, s_ref = oracle_prefill(x)
    _check("prefill_h8_t4k", o, st, o_ref, s_ref, TOL["bf16"])


@pytest.mark.parametrize("name,chains", [
    ("prefill_b4_h16_t16k", [(0, 0), (1, 7), (2, 12), (3, 15)]),
    ("prefill_h16_t128k", [(0, 0), (0, 11)]),
])
def test_full_size_sampled_chains(name, chains):
    w = WORKLOADS[name]
    log(f"[{name}] B{w.B} H{w.H} T{w.T} d{w.d_k} C{w.chunk} bf16, oracle on chains {chains}")
    x = workload_inputs(w)
    o, st = run_prefill(x, "bf16", w.chunk)
    o_ref, s_ref = _sampled(x, chains)
    o_gpu = np.stack([o[b, :, h] for b, h in chains], axis=1)[None]
    s_gpu = np.stack([st[b, h] for b, h in chains])[None]
    _check(name, o_gpu, s_gpu, o_ref, s_ref, TOL["bf16"])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(st))


def test_decode_b256_h16_1000_steps():
    import torch
    import gated_delta_rule_76_amd as kda

    w = WORKLOADS["decode_b256_h16"]
    steps, pool = w.decode_steps, 16
    log(f"[decode_b256_h16] B{w.B} H{w.H} d{w.d_k} x {steps} steps (pool {pool})")
    p = decode_pool(w.B, w.H, w.d_k, w.d_v, pool=pool, dtype=w.dtype, gate_c=w.gate_c,
                    s0_std=w.s0_std, seed=w.seed)
    dev = {n: to_dev(p[n], "bf16") for n in ("q", "k", "v", "alpha", "beta")}
    S = torch.from_numpy(p["S"]).cuda()
    o_hist = torch.empty((steps, w.B, w.H, w.d_v), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        i = t % pool
        kda.kda_decode_step(dev["q"][i], dev["k"][i], dev["v"][i], dev["alpha"][i], dev["beta"][i],
                            S, o=o_hist[t])
    torch.cuda.synchronize()
    heads = [(0, 0), (17, 3), (128, 9), (255, 15), (77, 8), (200, 1)]
    # The oracle runs the same 1000 steps as one T=1000 sequence per sampled head.
    seq = lambda a: np.stack([np.stack([a[t % pool, b, h] for t in range(steps)])
                              for b, h in heads], axis=1)[None]
    s0 = np.stack([p["S"][b, h] for b, h in heads])[None]
    o_ref, s_ref = oracle.kda_forward(seq(p["q"]), seq(p["k"]), seq(p["v"]), seq(p["alpha"]),
                                      seq(p["beta"]), s0)
    o_all = to_np(o_hist)
    o_gpu = np.stack([o_all[:, b, h] for b, h in heads], axis=1)[None]
    s_all = S.cpu().numpy()
    s_gpu = np.stack([s_all[b, h] for b, h in heads])[None]
    _check("decode_b256_h16", o_gpu, s_gpu, o_ref, s_ref, TOL["bf16"])
    assert np.all(np.isfinite(s_all))


# ------------------------------------------------------- shape / dtype sweep
SHAPES = [
    # dtype, d_k, d_v, C, B, T, H
    ("f32", 16, 16, 16, 1, 100, 2),
    ("f32", 32, 64, 32, 2, 77, 3),
    ("f32", 64, 32, 64, 1, 130, 2),
    ("f32", 128, 128, 32, 1, 96, 2),
    ("f32", 128, 16, 16, 1, 50, 1),
    ("f32", 64, 128, 64, 1, 64, 1),
    ("bf16", 128, 128, 64, 2, 333, 3),
    ("bf16", 128, 128, 32, 1, 200, 2),
    ("bf16", 128, 128, 16, 1, 100, 2),
    ("bf16", 64, 64, 64, 1, 257, 4),
    ("bf16", 16, 32, 16, 3, 45, 2),
    ("bf16", 32, 128, 32, 1, 129, 2),
    ("bf16", 128, 64, 64, 2, 1, 2),
    ("bf16", 128, 128, 64, 1, 63, 1),
    ("bf16", 128, 128, 64, 1, 65, 1),
    # enough (batch, head) chains that the state pass keeps 32-column value
    # blocks on a 256-CU device (fewer chains take 16-column blocks)
    ("bf16", 128, 128, 64, 4, 130, 10),
    ("bf16", 64, 64, 32, 5, 99, 14),
    ("f32", 64, 64, 32, 5, 70, 14),
]


@pytest.mark.parametrize("dtype,dk,dv,C,B,T,H", SHAPES)
def test_prefill_shapes(dtype, dk, dv, C, B, T, H):
    name = f"prefill {dtype} dk{dk} dv{dv} C{C} B{B} T{T} H{H}"
    log(f"[{name}]")
    x = prefill_inputs(B, T, H, dk, dv, dtype=dtype, gate_c=0.1, s0_std=0.05, seed=dk + dv + C + T)
    o, st = run_prefill(x, dtype, C)
    o_ref, s_ref = oracle_prefill(x)
    _check(name, o, st, o_ref, s_ref, TOL[dtype])


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 16, 16), ("f32", 128, 128), ("f32", 32, 128),
                                         ("bf16", 128, 128), ("bf16", 64, 16), ("bf16", 16, 64)])
def test_decode_shapes(dtype, dk, dv):
    import torch
    import gated_delta_rule_76_amd as kda

    B, H, steps = 5, 3, 20
    name = f"decode {dtype} dk{dk} dv{dv} B{B} H{H} x{steps}"
    log(f"[{name}]")
    p = decode_pool(B, H, dk, dv, pool=steps, dtype=dtype, gate_c=0.1, s0_std=0.05, seed=dk * dv)
    dev = {n: to_dev(p[n], dtype) for n in ("q", "k", "v", "alpha", "beta")}
    S = torch.from_numpy(p["S"]).cuda()
    outs = []
    for t in range(steps):
        outs.append(to_np(kda.kda_decode_step(dev["q"][t], dev["k"][t], dev["v"][t],
                                              dev["alpha"][t], dev["beta"][t], S)))
    torch.cuda.synchronize()
    tr = lambda a: np.moveaxis(a, 0, 1)  # [steps,B,H,..] -> [B,steps,H,..]
    o_ref, s_ref = oracle.kda_forward(tr(p["q"]), tr(p["k"]), tr(p["v"]), tr(p["alpha"]),
                                      tr(p["beta"]), p["S"])
    _check(name, tr(np.stack(outs)), S.cpu().numpy(), o_ref, s_ref, TOL[dtype])
