"""GPU parity of the AttnRes depth aggregation kernel against the fp64
oracle (page "Yanjiu KimiK3 ...", section 8)."""
import numpy as np
import pytest

from oracle.attnres import attnres_forward as oracle_attnres
from synth import attnres_inputs
from tests.gpu_harness import TOL, log, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,L,N,dk,d", [
    ("f32", 1, 7, 16, 8),          # one earlier layer: the output is that layer
    ("f32", 13, 33, 64, 520),      # L not a multiple of 4; d not a multiple of 2048
    ("f32", 64, 16, 128, 4096),
    ("bf16", 5, 17, 32, 264),
    ("bf16", 64, 64, 128, 4096),
    ("bf16", 1024, 3, 128, 64),    # the largest L
    ("bf16", 61, 128, 100, 2048),  # d_k not a multiple of 64
    ("bf16", 7, 9, 8, 8200),       # three sweeps of d, the last with one column group; one lane per key
    ("f32", 3, 5, 512, 16),        # fewer than four layers; one layer per wave step in the scores
    ("bf16", 4, 3, 256, 24),       # exactly one batch of four layers
])
def test_attnres_parity(dtype, L, N, dk, d):
    import torch
    import gated_delta_rule_76_amd as kda
    name = f"attnres {dtype} L{L} N{N} dk{dk} d{d}"
    log(f"[{name}]")
    x = attnres_inputs(L, N, dk, d, dtype=dtype, seed=L + N)
    out = kda.attnres_forward(to_dev(x["q"], dtype), to_dev(x["k"], dtype), to_dev(x["h"], dtype))
    torch.cuda.synchronize()
    ref = oracle_attnres(x["q"], x["k"], x["h"])
    e = rel_err(to_np(out), ref)
    log(f"  rel_err {e:.2e}")
    assert e <= TOL[dtype]
    if L == 1:
        assert np.array_equal(to_np(out), x["h"][0].astype(np.float64))


def test_attnres_deterministic():
    import torch
    import gated_delta_rule_76_amd as kda
    x = attnres_inputs(40, 50, 128, 1024, dtype="bf16", seed=9)
    q, k, h = (to_dev(x[n], "bf16") for n in ("q", "k", "h"))
    a = kda.attnres_forward(q, k, h)
    b = kda.attnres_forward(q, k, h)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attnres_tokens_are_independent():
    """A token's output depends only on its own q, k_i and h_i: the first 7
    tokens of a 50-token call equal a 7-token call on those tokens, bitwise."""
    import torch
    import gated_delta_rule_76_amd as kda
    log("[attnres token independence] bf16 L40 N50 dk128 d1024 vs its first 7 tokens")
    x = attnres_inputs(40, 50, 128, 1024, dtype="bf16", seed=11)
    full = kda.attnres_forward(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["h"], "bf16"))
    sub = kda.attnres_forward(to_dev(np.ascontiguousarray(x["q"][:7]), "bf16"),
                              to_dev(np.ascontiguousarray(x["k"][:, :7]), "bf16"),
                              to_dev(np.ascontiguousarray(x["h"][:, :7]), "bf16"))
    torch.cuda.synchronize()
    assert torch.equal(full[:7], sub)
