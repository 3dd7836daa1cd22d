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


def _diagnostics(name, o, st, o_ref, s_ref):
    """Per-(b, h) maximum of the relative error and the RMS-relative error of
    each tensor, logged next to the whole-tensor figure."""
    # o [B,T,H,d_v] -> per chain (b, h); S_T [B,H,d_k,d_v]
    do = np.abs(o - o_ref).max(axis=(1, 3)) / max(np.abs(o_ref).max(), 1e-300)
    ds = np.abs(st - s_ref).max(axis=(2, 3)) / max(np.abs(s_ref).max(), 1e-300)
    rms = lambda x, y: float(np.sqrt(np.mean((x - y) ** 2) / max(np.mean(y ** 2), 1e-300)))
    log(f"[{name}] per-chain max rel_err o={do.max():.3e} (median {np.median(do):.3e}), "
        f"S_T={ds.max():.3e}; rms-rel o={rms(o, o_ref):.3e} S_T={rms(st, s_ref):.3e}")


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
    _diagnostics("prefill_h8_t4k", o, st, o_ref, s_ref)


@pytest.mark.parametrize("name", ["prefill_b4_h16_t16k", "prefill_h16_t128k"])
def test_full_size_whole_tensor(name):
    """Every (batch, head) chain of the full-size workloads, in the launch
    configuration the benchmark times, against the oracle over the whole o and
    S_T tensors."""
    w = WORKLOADS[name]
    log(f"[{name}] B{w.B} H{w.H} T{w.T} d{w.d_k} C{w.chunk} bf16, oracle on all "
        f"{w.B * w.H} chains")
    x = workload_inputs(w)
    o, st = run_prefill(x, "bf16", w.chunk)
    log(f"[{name}] GPU done; oracle on {oracle.max_threads()} threads")
    o_ref, s_ref = oracle_prefill(x)
    del x
    _check(name, o, st, o_ref, s_ref, TOL["bf16"])
    _diagnostics(name, o, st, o_ref, s_ref)


def test_decode_b256_h16_1000_steps():
    """1000 consecutive decode steps, each with its own inputs, every head of
    every sequence compared with the oracle.  The oracle runs each block of
    steps as one sequence per head, carrying its fp64 state from block to
    block; o is compared over all 1000 steps as one tensor."""
    import torch
    import gated_delta_rule_76_amd as kda
    from synth import decode_state, decode_steps

    w = WORKLOADS["decode_b256_h16"]
    steps, block = w.decode_steps, 125
    log(f"[decode_b256_h16] B{w.B} H{w.H} d{w.d_k} x {steps} distinct steps, all heads")
    S_init = decode_state(w.B, w.H, w.d_k, w.d_v, s0_std=w.s0_std, seed=w.seed)
    S = torch.from_numpy(S_init).cuda()
    s_ref = S_init.astype(np.float64)
    err_o = ref_o = 0.0
    tr = lambda a: np.moveaxis(a, 0, 1)  # [steps,B,H,..] -> [B,steps,H,..]
    for first in range(0, steps, block):
        p = decode_steps(w.B, w.H, w.d_k, w.d_v, first, block, dtype=w.dtype, gate_c=w.gate_c,
                         seed=w.seed)
        dev = {n: to_dev(p[n], "bf16") for n in ("q", "k", "v", "alpha", "beta")}
        o_hist = torch.empty((block, w.B, w.H, w.d_v), dtype=torch.bfloat16, device="cuda")
        for t in range(block):
            kda.kda_decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["alpha"][t],
                                dev["beta"][t], S, o=o_hist[t])
        torch.cuda.synchronize()
        o_ref, s_ref = oracle.kda_forward(tr(p["q"]), tr(p["k"]), tr(p["v"]), tr(p["alpha"]),
                                          tr(p["beta"]), s_ref)
        o_gpu = tr(to_np(o_hist))
        assert np.all(np.isfinite(o_gpu))
        err_o = max(err_o, float(np.abs(o_gpu - o_ref).max()))
        ref_o = max(ref_o, float(np.abs(o_ref).max()))
        del dev, o_hist
        log(f"[decode_b256_h16] steps {first}..{first + block - 1} done")
    s_gpu = S.cpu().numpy().astype(np.float64)
    eo = err_o / ref_o
    es = rel_err(s_gpu, s_ref)
    log(f"[decode_b256_h16] rel_err o={eo:.3e} S={es:.3e} over all {w.B * w.H} heads "
        f"and {steps} steps (tol {TOL['bf16']:g})")
    assert np.all(np.isfinite(s_gpu))
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


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
    # more state-pass workgroups than CUs (128 chains x 4 value blocks): the
    # workgroups run in several rounds and never wait on one another
    ("bf16", 128, 128, 64, 8, 70, 16),
    # one 16-column value block per chain (d_v = 16) with the bf16 prep
    ("bf16", 128, 16, 64, 2, 150, 3),
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
