"""GPU parity of the gate / update-rule variants against the fp64 oracle.

Variants (page "Yanjiu KimiK3 ...", http://www.pwwt.cn/news/3763336/):
  gate "channel" : KDA's per-channel decay (section 4)
  gate "head"    : Gated DeltaNet's scalar forget gate (section 4)
  gate "none"    : no decay: the plain delta rule (section 3)
  rule "linear"  : no correction: the additive memory of section 2.1
Inputs are the seeded synthetic tensors; a per-head gate uses the first
channel of the drawn per-channel gate (same distribution).
"""
import numpy as np
import pytest

import oracle
from synth import decode_pool, prefill_inputs
from tests.gpu_harness import TOL, log, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

GATES = ["channel", "head", "none"]
RULES = ["delta", "linear"]


def _alpha(x, gate):
    return {"channel": x["alpha"], "head": np.ascontiguousarray(x["alpha"][..., 0]), "none": None}[gate]


def _prefill(x, dtype, chunk, gate, rule):
    import torch
    import gated_delta_rule_76_amd as kda
    q, k, v, be = (to_dev(x[n], dtype) for n in ("q", "k", "v", "beta"))
    a = _alpha(x, gate)
    al = None if a is None else to_dev(a, dtype)
    s0 = torch.from_numpy(np.ascontiguousarray(x["S0"], dtype=np.float32)).cuda()
    o, st = kda.kda_fwd_chunked(q, k, v, al, be, s0, chunk=chunk, gate=gate, rule=rule)
    torch.cuda.synchronize()
    return to_np(o), to_np(st)


CASES = [
    # dtype, d_k, d_v, C, B, T, H
    ("f32", 32, 32, 16, 1, 100, 2),
    ("f32", 64, 128, 32, 1, 77, 2),
    ("bf16", 128, 128, 64, 1, 200, 2),
    ("bf16", 64, 32, 32, 2, 129, 3),
]


@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("dtype,dk,dv,C,B,T,H", CASES)
def test_prefill_variant(gate, rule, dtype, dk, dv, C, B, T, H):
    name = f"prefill gate={gate} rule={rule} {dtype} dk{dk} dv{dv} C{C} B{B} T{T} H{H}"
    log(f"[{name}]")
    x = prefill_inputs(B, T, H, dk, dv, dtype=dtype, gate_c=0.1, s0_std=0.05, seed=7 + dk + T)
    o, st = _prefill(x, dtype, C, gate, rule)
    o_ref, s_ref = oracle.kda_forward(x["q"], x["k"], x["v"], _alpha(x, gate), x["beta"], x["S0"],
                                      gate=gate, rule=rule)
    eo, es = rel_err(o, o_ref), rel_err(st, s_ref)
    log(f"  rel_err o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_variant(gate, rule, dtype):
    import torch
    import gated_delta_rule_76_amd as kda
    B, H, dk, dv, steps = 4, 3, 128, 64, 12
    name = f"decode gate={gate} rule={rule} {dtype} B{B} H{H} dk{dk} dv{dv} x{steps}"
    log(f"[{name}]")
    p = decode_pool(B, H, dk, dv, pool=steps, dtype=dtype, gate_c=0.1, s0_std=0.05, seed=dk + 3)
    S = torch.from_numpy(p["S"]).cuda()
    Sref = p["S"].astype(np.float64)
    for i in range(steps):
        a = {"channel": p["alpha"][i], "head": np.ascontiguousarray(p["alpha"][i][..., 0]),
             "none": None}[gate]
        dev = {n: to_dev(p[n][i], dtype) for n in ("q", "k", "v", "beta")}
        al = None if a is None else to_dev(a, dtype)
        o = kda.kda_decode_step(dev["q"], dev["k"], dev["v"], al, dev["beta"], S, gate=gate, rule=rule)
        o_ref, Sref = oracle.kda_decode_step(p["q"][i], p["k"][i], p["v"][i], a, p["beta"][i], Sref,
                                             gate=gate, rule=rule)
        torch.cuda.synchronize()
        eo = rel_err(to_np(o), o_ref)
        assert eo <= TOL[dtype], (i, eo)
    es = rel_err(S.cpu().numpy(), Sref)
    log(f"  rel_err S after {steps} steps {es:.2e}")
    assert es <= TOL[dtype]


def test_gdn_prefill_h8_t4k_full():
    # Gated DeltaNet at the B=1, H=8, T=4096, d=128, C=64 bf16 prefill shape
    name = "prefill gate=head rule=delta bf16 B1 H8 T4096 d128 C64"
    log(f"[{name}]")
    x = prefill_inputs(1, 4096, 8, 128, 128, dtype="bf16", gate_c=0.1, s0_std=0.01, seed=1)
    o, st = _prefill(x, "bf16", 64, "head", "delta")
    o_ref, s_ref = oracle.kda_forward(x["q"], x["k"], x["v"], _alpha(x, "head"), x["beta"], x["S0"],
                                      gate="head")
    eo, es = rel_err(o, o_ref), rel_err(st, s_ref)
    log(f"  rel_err o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_head_gate_equals_broadcast_channel_gate_bitwise():
    # The per-head gate is the per-channel path with equal channels: feeding
    # the broadcast gate through the channel path gives the same bits.
    import torch
    import gated_delta_rule_76_amd as kda
    x = prefill_inputs(1, 150, 2, 128, 128, dtype="bf16", gate_c=0.1, s0_std=0.05, seed=5)
    xa = dict(x)
    xa["alpha"] = np.ascontiguousarray(np.broadcast_to(x["alpha"][..., :1], x["alpha"].shape))
    o1, s1 = _prefill(xa, "bf16", 64, "head", "delta")
    o2, s2 = _prefill(xa, "bf16", 64, "channel", "delta")
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


# ---------------------------------------------------------- fused prologue
from synth import raw_prefill_inputs  # noqa: E402


def _graw(x, gate):
    return {"channel": x["g_raw"], "head": np.ascontiguousarray(x["g_raw"][..., 0]), "none": None}[gate]


FUSED = [
    # dtype, d_k, d_v, C, B, T, H, gate, rule
    ("f32", 32, 32, 16, 1, 100, 2, "channel", "delta"),
    ("f32", 64, 64, 32, 1, 70, 2, "head", "linear"),
    ("bf16", 128, 128, 64, 1, 200, 2, "channel", "delta"),
    ("bf16", 128, 128, 64, 2, 130, 2, "head", "delta"),
    ("bf16", 64, 128, 32, 1, 99, 3, "none", "delta"),
    ("bf16", 16, 32, 16, 1, 50, 2, "channel", "linear"),
]


@pytest.mark.parametrize("dtype,dk,dv,C,B,T,H,gate,rule", FUSED)
def test_prefill_fused_prologue(dtype, dk, dv, C, B, T, H, gate, rule):
    import torch
    import gated_delta_rule_76_amd as kda
    name = f"prefill fused gate={gate} rule={rule} {dtype} dk{dk} dv{dv} C{C} B{B} T{T} H{H}"
    log(f"[{name}]")
    x = raw_prefill_inputs(B, T, H, dk, dv, dtype=dtype, s0_std=0.05, seed=dk + T)
    c = 0.1
    q, k, v, b = (to_dev(x[n], dtype) for n in ("q_raw", "k_raw", "v", "b_raw"))
    g = _graw(x, gate)
    gd = None if g is None else to_dev(g, dtype)
    s0 = torch.from_numpy(x["S0"]).cuda()
    o, st = kda.kda_fwd_chunked_fused(q, k, v, gd, b, s0, gate_scale=c, chunk=C, gate=gate, rule=rule)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.kda_forward_fused(x["q_raw"], x["k_raw"], x["v"], g, x["b_raw"], x["S0"],
                                            gate_scale=c, gate=gate, rule=rule)
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(st), s_ref)
    log(f"  rel_err o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,gate", [("f32", "channel"), ("bf16", "channel"), ("bf16", "head"),
                                        ("bf16", "none")])
def test_decode_fused_prologue(dtype, gate):
    import torch
    import gated_delta_rule_76_amd as kda
    B, H, dk, dv, steps, c = 4, 3, 128, 128, 8, 0.05
    log(f"[decode fused gate={gate} {dtype} B{B} H{H} x{steps}]")
    x = raw_prefill_inputs(B, steps, H, dk, dv, dtype=dtype, s0_std=0.05, seed=11)
    S = torch.from_numpy(x["S0"]).cuda()
    Sref = x["S0"].astype(np.float64)
    for i in range(steps):
        sl = {n: np.ascontiguousarray(x[n][:, i]) for n in ("q_raw", "k_raw", "v", "g_raw", "b_raw")}
        g = {"channel": sl["g_raw"], "head": np.ascontiguousarray(sl["g_raw"][..., 0]), "none": None}[gate]
        d = {n: to_dev(sl[n], dtype) for n in ("q_raw", "k_raw", "v", "b_raw")}
        o = kda.kda_decode_step_fused(d["q_raw"], d["k_raw"], d["v"], None if g is None else to_dev(g, dtype),
                                      d["b_raw"], S, gate_scale=c, gate=gate)
        q, k, a, b = oracle.input_prologue(sl["q_raw"], sl["k_raw"], g, sl["b_raw"], c, gate)
        o_ref, Sref = oracle.kda_decode_step(q, k, sl["v"], a, b, Sref, gate=gate)
        torch.cuda.synchronize()
        assert rel_err(to_np(o), o_ref) <= TOL[dtype]
    es = rel_err(S.cpu().numpy(), Sref)
    log(f"  rel_err S after {steps} steps {es:.2e}")
    assert es <= TOL[dtype]


def test_prefill_fused_prologue_32_column_blocks():
    """The fused entry point with enough chains (40) that the state pass takes
    32-column value blocks on a 256-CU device; the oracle checks two chains."""
    import torch
    import gated_delta_rule_76_amd as kda
    B, T, H, c = 4, 2048, 10, 0.05
    log(f"[prefill fused gate=channel bf16 dk128 dv128 C64 B{B} T{T} H{H}, oracle on 2 chains]")
    x = raw_prefill_inputs(B, T, H, 128, 128, dtype="bf16", s0_std=0.01, seed=77)
    q, k, v, g, b = (to_dev(x[n], "bf16") for n in ("q_raw", "k_raw", "v", "g_raw", "b_raw"))
    s0 = torch.from_numpy(x["S0"]).cuda()
    o, st = kda.kda_fwd_chunked_fused(q, k, v, g, b, s0, gate_scale=c, chunk=64)
    torch.cuda.synchronize()
    o, st = to_np(o), to_np(st)
    for bb, hh in ((0, 0), (3, 9)):
        sl = lambda a: np.ascontiguousarray(a[bb:bb + 1, :, hh:hh + 1])
        o_ref, s_ref = oracle.kda_forward_fused(sl(x["q_raw"]), sl(x["k_raw"]), sl(x["v"]), sl(x["g_raw"]),
                                                sl(x["b_raw"]), np.ascontiguousarray(x["S0"][bb:bb + 1, hh:hh + 1]),
                                                gate_scale=c)
        eo = rel_err(o[bb:bb + 1, :, hh:hh + 1], o_ref)
        es = rel_err(st[bb:bb + 1, hh:hh + 1], s_ref)
        log(f"  chain ({bb},{hh}): rel_err o {eo:.2e}  S_T {es:.2e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(st))


@pytest.mark.parametrize("gate,rule", [("head", "delta"), ("channel", "linear")])
def test_variants_32_column_blocks(gate, rule):
    """The per-head gate and the uncorrected write with enough chains (40) that
    the state pass takes 32-column value blocks on a 256-CU device; the oracle
    checks two chains."""
    B, T, H = 4, 1000, 10
    log(f"[prefill gate={gate} rule={rule} bf16 dk128 dv128 C64 B{B} T{T} H{H}, oracle on 2 chains]")
    x = prefill_inputs(B, T, H, 128, 128, dtype="bf16", gate_c=0.05, s0_std=0.01, seed=88)
    o, st = _prefill(x, "bf16", 64, gate, rule)
    a = _alpha(x, gate)
    for bb, hh in ((0, 0), (3, 9)):
        sl = lambda arr: None if arr is None else np.ascontiguousarray(arr[bb:bb + 1, :, hh:hh + 1])
        o_ref, s_ref = oracle.kda_forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(a), sl(x["beta"]),
                                          np.ascontiguousarray(x["S0"][bb:bb + 1, hh:hh + 1]),
                                          gate=gate, rule=rule)
        eo = rel_err(o[bb:bb + 1, :, hh:hh + 1], o_ref)
        es = rel_err(st[bb:bb + 1, hh:hh + 1], s_ref)
        log(f"  chain ({bb},{hh}): rel_err o {eo:.2e}  S_T {es:.2e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


# ---------------------------------------------------- strong decays, range edge
def _chunk_log_decay(alpha, C):
    """Per (batch, chunk, head, channel): the sum of log alpha over the
    chunk's tokens, in fp64 (-inf where an alpha is 0)."""
    a = np.asarray(alpha, dtype=np.float64)
    B, T, H, D = a.shape
    n = (T + C - 1) // C
    pad = np.ones((B, n * C - T, H, D))
    with np.errstate(divide="ignore"):
        la = np.log(np.concatenate([a, pad], axis=1))
    return la.reshape(B, n, C, H, D).sum(axis=2)


# In range means every chunk's decay stays above e^-80 in every channel (the
# kernels need 2^-126 ~ e^-87.3; the margin keeps fp32 rounding away from it).
STRONG = [
    # dtype, d_k, d_v, C, B, T, H, gate_scale
    ("bf16", 128, 128, 64, 2, 300, 2, 1.0),
    ("bf16", 128, 128, 16, 1, 250, 3, 2.0),
    ("bf16", 64, 64, 32, 2, 200, 2, 1.5),
    ("f32", 64, 64, 16, 1, 150, 2, 3.0),
]


@pytest.mark.parametrize("dtype,dk,dv,C,B,T,H,c", STRONG)
def test_fused_strong_gates_in_range(dtype, dk, dv, C, B, T, H, c):
    """Fused prologue with gate scales of 1 to 3 (per-token decays down to
    e^-10 and below): where every chunk's decay stays in range, the chunked
    prefill matches the oracle."""
    import torch
    import gated_delta_rule_76_amd as kda
    log(f"[strong gates] fused {dtype} dk{dk} dv{dv} C{C} B{B} T{T} H{H} gate_scale {c}")
    x = raw_prefill_inputs(B, T, H, dk, dv, dtype=dtype, s0_std=0.05, seed=int(c * 10) + C)
    _, _, alpha, _ = oracle.input_prologue(x["q_raw"], x["k_raw"], x["g_raw"], x["b_raw"], c)
    lmin = float(_chunk_log_decay(alpha, C).min())
    log(f"  smallest chunk log-decay {lmin:.1f}; smallest alpha {float(alpha.min()):.2e}")
    assert lmin > -80.0, "test inputs must stay inside the chunked form's range"
    q, k, v, g, b = (to_dev(x[n], dtype) for n in ("q_raw", "k_raw", "v", "g_raw", "b_raw"))
    s0 = torch.from_numpy(x["S0"]).cuda()
    o, st = kda.kda_fwd_chunked_fused(q, k, v, g, b, s0, gate_scale=c, chunk=C)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.kda_forward_fused(x["q_raw"], x["k_raw"], x["v"], x["g_raw"], x["b_raw"],
                                            x["S0"], gate_scale=c)
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(st), s_ref)
    log(f"  rel_err o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,C", [("bf16", 64), ("bf16", 16), ("f32", 32)])
def test_near_zero_decays_in_range(dtype, C):
    """Single tokens whose gate nearly closes (alpha = 1e-12 in some channels)
    inside otherwise ordinary gates: in range, so the oracle is matched."""
    log(f"[near-zero decays] {dtype} dk128 C{C} B2 T260 H2")
    x = prefill_inputs(2, 260, 2, 128, 128, dtype=dtype, gate_c=0.1, s0_std=0.05, seed=41 + C)
    rng = np.random.default_rng(5)
    a = x["alpha"]
    for t in rng.choice(260, size=6, replace=False):
        ch = rng.choice(128, size=40, replace=False)
        a[:, t, :, ch] = 1e-12
    if dtype == "bf16":
        from synth import round_to_bf16
        x["alpha"] = round_to_bf16(a)
    assert float(_chunk_log_decay(x["alpha"], C).min()) > -80.0
    o, st = _prefill(x, dtype, C, "channel", "delta")
    o_ref, s_ref = oracle.kda_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    eo, es = rel_err(o, o_ref), rel_err(st, s_ref)
    log(f"  rel_err o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,C", [("bf16", 64), ("f32", 32)])
def test_out_of_range_chunk_turns_its_chain_nan(dtype, C):
    """An alpha of exactly 0 puts its chunk outside the chunked form's range.
    The documented outcome: that chain's outputs from the start of the chunk
    on, and its final state, are NaN; earlier outputs and every other chain
    still match the oracle (which handles alpha = 0 exactly)."""
    B, T, H = 2, 300, 3
    log(f"[out of range] {dtype} dk128 C{C} B{B} T{T} H{H}, alpha = 0 at (b=1, t=150, h=2)")
    x = prefill_inputs(B, T, H, 128, 128, dtype=dtype, gate_c=0.1, s0_std=0.05, seed=43)
    t0, n0 = 150, (150 // C) * C
    x["alpha"][1, t0, 2, 7] = 0.0
    o, st = _prefill(x, dtype, C, "channel", "delta")
    o_ref, s_ref = oracle.kda_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    assert np.all(np.isnan(o[1, n0:, 2])) and np.all(np.isnan(st[1, 2]))
    assert np.all(np.isfinite(o[1, :n0, 2]))
    good_o = np.concatenate([o[0].reshape(-1), o[1, :, :2].reshape(-1), o[1, :n0, 2].reshape(-1)])
    ref_o = np.concatenate([o_ref[0].reshape(-1), o_ref[1, :, :2].reshape(-1),
                            o_ref[1, :n0, 2].reshape(-1)])
    good_s = np.concatenate([st[0].reshape(-1), st[1, :2].reshape(-1)])
    ref_s = np.concatenate([s_ref[0].reshape(-1), s_ref[1, :2].reshape(-1)])
    eo, es = rel_err(good_o, ref_o), rel_err(good_s, ref_s)
    log(f"  other outputs: rel_err o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_fused_gates_beyond_range_are_nan():
    """Gate scale 3 at chunk 64 takes every chunk's decay below e^-87: every
    output and the final state come back NaN (the documented outcome), and
    the same inputs at chunk 16 stay in range and match the oracle."""
    import torch
    import gated_delta_rule_76_amd as kda
    B, T, H, d, c = 1, 192, 2, 64, 3.0
    log(f"[beyond range] fused bf16 d{d} B{B} T{T} H{H} gate_scale {c}, chunks 64 and 16")
    x = raw_prefill_inputs(B, T, H, d, d, dtype="bf16", s0_std=0.05, seed=47)
    _, _, alpha, _ = oracle.input_prologue(x["q_raw"], x["k_raw"], x["g_raw"], x["b_raw"], c)
    assert float(_chunk_log_decay(alpha, 64).max()) < -95.0
    assert float(_chunk_log_decay(alpha, 16).min()) > -80.0
    q, k, v, g, b = (to_dev(x[n], "bf16") for n in ("q_raw", "k_raw", "v", "g_raw", "b_raw"))
    s0 = torch.from_numpy(x["S0"]).cuda()
    o64, st64 = kda.kda_fwd_chunked_fused(q, k, v, g, b, s0, gate_scale=c, chunk=64)
    o16, st16 = kda.kda_fwd_chunked_fused(q, k, v, g, b, s0, gate_scale=c, chunk=16)
    torch.cuda.synchronize()
    assert torch.isnan(o64.float()).all().item() and torch.isnan(st64).all().item()
    o_ref, s_ref = oracle.kda_forward_fused(x["q_raw"], x["k_raw"], x["v"], x["g_raw"], x["b_raw"],
                                            x["S0"], gate_scale=c)
    eo, es = rel_err(to_np(o16), o_ref), rel_err(to_np(st16), s_ref)
    log(f"  chunk 16: rel_err o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
