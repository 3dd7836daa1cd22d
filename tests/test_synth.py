"""Seeded input generators: determinism, bf16 rounding and value ranges."""
import numpy as np
import torch

from synth import WORKLOADS, decode_pool, orthonormal_key_set, prefill_inputs, round_to_bf16


def test_same_seed_same_bytes():
    a = prefill_inputs(1, 33, 2, 16, 8, dtype="bf16", seed=7)
    b = prefill_inputs(1, 33, 2, 16, 8, dtype="bf16", seed=7)
    for n in ("q", "k", "v", "alpha", "beta", "S0"):
        assert a[n].tobytes() == b[n].tobytes()
    c = prefill_inputs(1, 33, 2, 16, 8, dtype="bf16", seed=8)
    assert a["q"].tobytes() != c["q"].tobytes()


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-30, 30, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.0e38, 1e-40], dtype=np.float32)])
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_value_ranges_and_exactness():
    x = prefill_inputs(2, 64, 4, 128, 128, dtype="bf16", gate_c=0.05, seed=2)
    for n in ("q", "k", "v", "alpha", "beta"):
        np.testing.assert_array_equal(round_to_bf16(x[n]), x[n])
    nk = np.linalg.norm(x["k"].astype(np.float64), axis=-1)
    assert np.all(np.abs(nk - 1) < 2e-2)
    assert np.all((x["alpha"] > 0) & (x["alpha"] <= 1))
    assert np.all((x["beta"] > 0) & (x["beta"] < 1))
    assert x["S0"].dtype == np.float32 and abs(x["S0"].std() - 0.01) < 1e-3


def test_decode_pool_shapes():
    p = decode_pool(4, 2, 16, 8, pool=3)
    assert p["q"].shape == (3, 4, 2, 16) and p["v"].shape == (3, 4, 2, 8)
    assert p["beta"].shape == (3, 4, 2) and p["S"].shape == (4, 2, 16, 8)


def test_decode_steps_are_distinct_and_drawn_piecewise():
    from synth import decode_state, decode_steps
    whole = decode_steps(3, 2, 16, 8, 0, 6, dtype="bf16")
    part = decode_steps(3, 2, 16, 8, 4, 2, dtype="bf16")
    for n in whole:
        np.testing.assert_array_equal(whole[n][4:], part[n])
        assert not np.array_equal(whole[n][0], whole[n][1])
        np.testing.assert_array_equal(round_to_bf16(whole[n]), whole[n])
    assert whole["alpha"].shape == (6, 3, 2, 16) and whole["beta"].shape == (6, 3, 2)
    assert np.all((whole["alpha"] > 0) & (whole["alpha"] <= 1))
    s = decode_state(3, 2, 16, 8)
    assert s.shape == (3, 2, 16, 8) and s.dtype == np.float32


def test_orthonormal_keys_exact():
    for d, kind in [(16, "hadamard"), (64, "hadamard"), (32, "onehot"), (8, "signed")]:
        K = orthonormal_key_set(d, kind).astype(np.float64)
        np.testing.assert_allclose(K @ K.T, np.eye(d), atol=1e-15)
        np.testing.assert_array_equal(round_to_bf16(K.astype(np.float32)), K.astype(np.float32))


def test_workload_table():
    assert set(WORKLOADS) == {"tiny_f32", "prefill_h8_t4k", "prefill_b4_h16_t16k",
                              "prefill_h16_t128k", "decode_b256_h16"}
    assert WORKLOADS["prefill_h16_t128k"].T // WORKLOADS["prefill_h16_t128k"].chunk == 2048
