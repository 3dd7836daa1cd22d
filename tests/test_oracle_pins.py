"""Pins for the fp64 oracle: each check is fixed by the pages or by mathematics,
not by re-running the oracle's own formula.

Passages (page "Yanjiu KimiK3 ...", http://www.pwwt.cn/news/3763336/):
  section 2.1 : state S in R^{d_k x d_v}; plain write S += k v^T; read o = S^T q
  section 3   : delta rule, error form S += beta k (v - S^T k)^T and the
                equivalent projection form (I - beta k k^T) S + beta k v^T;
                a newer value overwrites the old one stored under the same key
  section 4   : KDA, S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
  section 5   : transition A_i = (I - beta_i k_i k_i^T) Diag(alpha_i); a write at
                j reaches t through A_t ... A_{j+1}
  section 6   : affine recurrence S_t = A_t S_{t-1} + B_t; chunking; P = D - K W^T
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import orthonormal_key_set, prefill_inputs
from tests.chunked_model import chunk_factors, chunked_forward
from tests.golden.load import overwrite_recall


def _rel(x, y):
    return np.max(np.abs(np.asarray(x) - np.asarray(y))) / max(np.max(np.abs(y)), 1e-300)


def _rand_inputs(rng, B, T, H, dk, dv, normalise=True, beta_range=(0.0, 1.0)):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if normalise:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal((B, T, H, dk))) * 0.3)
    beta = rng.uniform(*beta_range, size=(B, T, H))
    S0 = 0.1 * rng.standard_normal((B, H, dk, dv))
    return q, k, v, alpha, beta, S0


# --------------------------------------------------------------------------
# P1: alpha = 1, beta = 1, orthonormal keys, S0 = 0 -> exact recall of the
#     last value written under each key (sections 2.1 and 3, overwrite rule).
# --------------------------------------------------------------------------
def test_p1_golden_onehot_overwrite():
    g = overwrite_recall()
    T, d = len(g["keys"]), 4
    E = np.eye(d)
    k = E[g["keys"]][None, :, None, :]
    q = E[g["queries"]][None, :, None, :]
    v = g["v"][None, :, None, :]
    alpha = np.ones_like(k)
    beta = np.ones((1, T, 1))
    o, ST = oracle.kda_forward(q, k, v, alpha, beta)
    np.testing.assert_array_equal(o[0, :, 0], g["o_expected"])
    np.testing.assert_array_equal(ST[0, 0], g["S_expected"])


@pytest.mark.parametrize("kind", ["qr", "hadamard"])
def test_p1_orthonormal_recall(kind):
    rng = np.random.default_rng(11)
    dk, dv, T = 16, 5, 200
    if kind == "qr":
        keys, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        keys = keys.T
    else:
        keys = orthonormal_key_set(dk, "hadamard").astype(np.float64)
    kid = rng.integers(0, dk, size=T)
    qid = rng.integers(0, dk, size=T)
    v = rng.standard_normal((T, dv))
    last = {}
    expect = np.zeros((T, dv))
    for t in range(T):
        last[kid[t]] = v[t]
        expect[t] = last.get(qid[t], np.zeros(dv))
    o, ST = oracle.kda_forward(keys[qid][None, :, None], keys[kid][None, :, None], v[None, :, None],
                               np.ones((1, T, 1, dk)), np.ones((1, T, 1)))
    assert np.max(np.abs(o[0, :, 0] - expect)) < 1e-12
    S_expect = sum(np.outer(keys[m], last[m]) for m in last)
    assert np.max(np.abs(ST[0, 0] - S_expect)) < 1e-12


# --------------------------------------------------------------------------
# P2: beta = 0 writes nothing.  With alpha = 1, S_T = S0 and o_t = S0^T q_t.
#     P2b: with general alpha, S_T = Diag(prod_t alpha_t) S0 and
#     o_t = S0^T (gamma_t * q_t), gamma_t = prod_{s<=t} alpha_s  (section 4:
#     Diag(alpha_t) scales the key channels of the old state).
# --------------------------------------------------------------------------
def test_p2_beta_zero_alpha_one_keeps_state():
    rng = np.random.default_rng(2)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 2, 37, 3, 8, 6)
    o, ST = oracle.kda_forward(q, k, v, np.ones_like(alpha), np.zeros_like(beta), S0)
    np.testing.assert_array_equal(ST, S0)
    expect = np.einsum("bthi,bhij->bthj", q, S0)
    assert _rel(o, expect) < 1e-14


def test_p2b_beta_zero_pure_decay():
    rng = np.random.default_rng(3)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, 29, 2, 7, 5)
    o, ST = oracle.kda_forward(q, k, v, alpha, np.zeros_like(beta), S0)
    gamma = np.cumprod(alpha, axis=1)
    assert _rel(ST, gamma[:, -1][..., None] * S0) < 1e-14
    expect = np.einsum("bthi,bhij->bthj", gamma * q, S0)
    assert _rel(o, expect) < 1e-13


# --------------------------------------------------------------------------
# P3a: alpha = 1 gives the plain delta rule; code it independently in both
#      algebraic forms of section 3.
# --------------------------------------------------------------------------
def test_p3a_alpha_one_is_delta_rule_both_forms():
    rng = np.random.default_rng(4)
    dk, dv, T = 6, 9, 50
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, T, 1, dk, dv)
    o, ST = oracle.kda_forward(q, k, v, np.ones_like(alpha), beta, S0)
    S_err = S0[0, 0].copy()
    S_proj = S0[0, 0].copy()
    o_err = np.zeros((T, dv)); o_proj = np.zeros((T, dv))
    for t in range(T):
        kt, vt, qt, bt = k[0, t, 0], v[0, t, 0], q[0, t, 0], beta[0, t, 0]
        e = vt - S_err.T @ kt                                  # prediction error
        S_err = S_err + bt * np.outer(kt, e)                    # error-form write
        S_proj = (np.eye(dk) - bt * np.outer(kt, kt)) @ S_proj + bt * np.outer(kt, vt)
        o_err[t] = S_err.T @ qt
        o_proj[t] = S_proj.T @ qt
    assert _rel(o[0, :, 0], o_err) < 1e-13
    assert _rel(o[0, :, 0], o_proj) < 1e-13
    assert _rel(ST[0, 0], S_proj) < 1e-13


# --------------------------------------------------------------------------
# P3b: with the correction removed and alpha = beta = 1, the write is the
#      plain linear memory S += k v^T of section 2.1, so o = tril(Q K^T) V.
# P3c: correction removed, general alpha/beta:
#      o = tril((Q*Gamma)(K/Gamma)^T) Diag(beta) V  (+ the decayed S0 term),
#      which pins that alpha scales KEY channels with inclusive cumulative decay.
# --------------------------------------------------------------------------
def test_p3b_linear_attention():
    rng = np.random.default_rng(5)
    T, dk, dv = 40, 8, 3
    q, k, v, alpha, beta, _ = _rand_inputs(rng, 1, T, 1, dk, dv)
    o, ST = oracle.kda_forward(q, k, v, np.ones_like(alpha), np.ones_like(beta), None,
                               no_correction=True)
    Q, K, V = q[0, :, 0], k[0, :, 0], v[0, :, 0]
    assert _rel(o[0, :, 0], np.tril(Q @ K.T) @ V) < 1e-13
    assert _rel(ST[0, 0], K.T @ V) < 1e-13


def test_p3c_gated_linear_attention_closed_form():
    rng = np.random.default_rng(6)
    T, dk, dv = 33, 5, 4
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, T, 1, dk, dv)
    o, ST = oracle.kda_forward(q, k, v, alpha, beta, S0, no_correction=True)
    Q, K, V, G = q[0, :, 0], k[0, :, 0], v[0, :, 0], np.cumprod(alpha[0, :, 0], axis=0)
    expect = np.tril((Q * G) @ (K / G).T) @ np.diag(beta[0, :, 0]) @ V + (Q * G) @ S0[0, 0]
    assert _rel(o[0, :, 0], expect) < 1e-12


# --------------------------------------------------------------------------
# P4: brute force with explicit dense transitions A_t = (I - b k k^T) Diag(a)
#     and writes B_t = b k v^T (sections 5 and 6), in two forms: the affine
#     recurrence S_t = A_t S_{t-1} + B_t and the path-product sum
#     S_T = (A_T..A_1) S0 + sum_j (A_T..A_{j+1}) B_j.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_p4_brute_force_transition_products(T):
    rng = np.random.default_rng(100 + T)
    dk, dv = 4, 3
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, T, 1, dk, dv, normalise=False,
                                            beta_range=(-0.5, 1.5))
    o, ST = oracle.kda_forward(q, k, v, alpha, beta, S0)
    At = [(np.eye(dk) - beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0])) @ np.diag(alpha[0, t, 0])
          for t in range(T)]
    Bt = [beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0]) for t in range(T)]
    S = S0[0, 0]
    for t in range(T):
        S = At[t] @ S + Bt[t]
        assert _rel(o[0, t, 0], S.T @ q[0, t, 0]) < 1e-13
    assert _rel(ST[0, 0], S) < 1e-13
    # path-product form
    def path(t_hi, j):  # A_{t_hi} ... A_{j+1}  (1-based t_hi, j)
        M = np.eye(dk)
        for i in range(j, t_hi):
            M = At[i] @ M
        return M
    S_sum = path(T, 0) @ S0[0, 0] + sum(path(T, j + 1) @ Bt[j] for j in range(T))
    assert _rel(ST[0, 0], S_sum) < 1e-13


def _exact_kda(q, k, v, alpha, beta, S0):
    """Exact rational recurrence in the projection form of section 4."""
    T, dk = len(q), len(q[0])
    dv = len(v[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        # Diag(alpha) S
        Sd = [[alpha[t][i] * S[i][j] for j in range(dv)] for i in range(dk)]
        # (I - beta k k^T) Sd + beta k v^T
        kS = [sum(k[t][i] * Sd[i][j] for i in range(dk)) for j in range(dv)]
        S = [[Sd[i][j] - beta[t] * k[t][i] * kS[j] + beta[t] * k[t][i] * v[t][j]
              for j in range(dv)] for i in range(dk)]
        outs.append([sum(S[i][j] * q[t][i] for i in range(dk)) for j in range(dv)])
    return outs, S


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p4_exact_rational(seed):
    rng = np.random.default_rng(seed)
    T, dk, dv = 8, 4, 3
    fr = lambda lo, hi, den: Fraction(int(rng.integers(lo, hi)), den)
    q = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    k = [[fr(-4, 5, 4) for _ in range(dk)] for _ in range(T)]       # not normalised
    v = [[fr(-16, 17, 4) for _ in range(dv)] for _ in range(T)]
    alpha = [[fr(0, 9, 8) for _ in range(dk)] for _ in range(T)]    # includes alpha = 0
    beta = [fr(0, 5, 4) for _ in range(T)]
    S0 = [[fr(-4, 5, 16) for _ in range(dv)] for _ in range(dk)]
    o_ex, S_ex = _exact_kda(q, k, v, alpha, beta, S0)
    f = lambda x: np.array(x, dtype=np.float64)
    o, ST = oracle.kda_forward(f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None],
                               f(alpha)[None, :, None], f(beta)[None, :, None], f(S0)[None, None])
    assert _rel(o[0, :, 0], f(o_ex)) < 1e-14
    assert _rel(ST[0, 0], f(S_ex)) < 1e-14


def test_alpha_zero_forgets_everything():
    # alpha_t = 0 wipes the old state: S_t = beta_t k_t v_t^T, o_t = beta_t (k_t . q_t) v_t.
    rng = np.random.default_rng(8)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, 6, 1, 5, 4)
    o, ST = oracle.kda_forward(q, k, v, np.zeros_like(alpha), beta, S0)
    kt, qt, vt, bt = k[0, :, 0], q[0, :, 0], v[0, :, 0], beta[0, :, 0]
    expect = (bt * np.sum(kt * qt, axis=1))[:, None] * vt
    assert _rel(o[0, :, 0], expect) < 1e-14
    assert _rel(ST[0, 0], bt[-1] * np.outer(kt[-1], vt[-1])) < 1e-14


# --------------------------------------------------------------------------
# P5/P7: the chunked design model equals the token recurrence for any chunk
# size, and the chunk's transition product has the WY form
# Diag(gamma_C) - Kbar^T W (section 6.2, P = D - K W^T).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_p5_chunk_size_invariance(C):
    rng = np.random.default_rng(9)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, 100, 2, 16, 12)
    o_ref, S_ref = oracle.kda_forward(q, k, v, alpha, beta, S0)
    o, ST = chunked_forward(q, k, v, alpha, beta, S0, C=C)
    assert _rel(o, o_ref) < 1e-12
    assert _rel(ST, S_ref) < 1e-12


def test_p7_wy_identity():
    rng = np.random.default_rng(10)
    C, dk = 16, 8
    K = rng.standard_normal((C, dk)); K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q = rng.standard_normal((C, dk))
    Al = np.exp(-np.logaddexp(0, rng.standard_normal((C, dk))) * 0.2)
    Bt = rng.uniform(0, 1, C)
    f = chunk_factors(K, Al, Bt, Q)
    prod = np.eye(dk)
    for r in range(C):
        prod = (np.eye(dk) - Bt[r] * np.outer(K[r], K[r])) @ np.diag(Al[r]) @ prod
    assert np.max(np.abs(np.diag(f["gamma_C"]) - f["Kbar"].T @ f["W"] - prod)) < 1e-13


# --------------------------------------------------------------------------
# P6: split / resume and decode == prefill on the oracle itself (exactness of
# the carried state; the GPU versions of these are the real checks).
# --------------------------------------------------------------------------
def test_p6_decode_steps_equal_prefill():
    rng = np.random.default_rng(12)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 2, 10, 3, 6, 4)
    o_ref, S_ref = oracle.kda_forward(q, k, v, alpha, beta, S0)
    S = S0
    for t in range(10):
        o_t, S = oracle.kda_decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S)
        np.testing.assert_array_equal(o_t, o_ref[:, t])
    np.testing.assert_array_equal(S, S_ref)


# --------------------------------------------------------------------------
# P8: contraction.  For beta in [0,1], |k| <= 1, alpha <= 1 every transition
# has spectral norm <= 1, so |S_t|_F <= |S_{t-1}|_F + beta_t |k_t| |v_t|.
# --------------------------------------------------------------------------
def test_p8_contraction_bound():
    rng = np.random.default_rng(13)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, 300, 1, 8, 8)
    S = S0[:, 0]
    for t in range(300):
        _, Sn = oracle.kda_decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], S[:, None])
        Sn = Sn[:, 0]
        bound = np.linalg.norm(S) + beta[0, t, 0] * np.linalg.norm(k[0, t, 0]) * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(Sn) <= bound * (1 + 1e-12)
        S = Sn


def test_layout_and_chain_independence():
    # (b, h) chains are independent: permuting heads permutes outputs, and a
    # chain computed alone equals the same chain inside a batch.
    x = prefill_inputs(2, 20, 3, 8, 8, dtype="f32", gate_c=0.1, s0_std=0.01, seed=5)
    o, ST = oracle.kda_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    perm = [2, 0, 1]
    o2, ST2 = oracle.kda_forward(x["q"][:, :, perm], x["k"][:, :, perm], x["v"][:, :, perm],
                                 x["alpha"][:, :, perm], x["beta"][:, :, perm], x["S0"][:, perm])
    np.testing.assert_array_equal(o2, o[:, :, perm])
    np.testing.assert_array_equal(ST2, ST[:, perm])
    o1, ST1 = oracle.kda_forward(x["q"][1:, :, 2:], x["k"][1:, :, 2:], x["v"][1:, :, 2:],
                                 x["alpha"][1:, :, 2:], x["beta"][1:, :, 2:], x["S0"][1:, 2:])
    np.testing.assert_array_equal(o1, o[1:, :, 2:])


def test_no_correction_differs_from_delta():
    # A planted-mistake guard: dropping the prediction term must change the
    # result (otherwise P3a would not be able to see it).
    rng = np.random.default_rng(14)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, 20, 1, 4, 4)
    o1, _ = oracle.kda_forward(q, k, v, alpha, beta, S0)
    o2, _ = oracle.kda_forward(q, k, v, alpha, beta, S0, no_correction=True)
    assert _rel(o1, o2) > 1e-3


# --------------------------------------------------------------------------
# Gate and rule variants.
#   Gated DeltaNet (section 4, the scalar forget gate KDA refines):
#     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
#     alpha_t one scalar per (token, head), coded here with dense matrices in
#     exactly the page's order (gate outside the erase), independently of the
#     oracle's per-channel loop.
#   No gate with the delta rule is section 3's delta rule; no gate, no
#   correction and beta = 1 is section 2.1's S_t = S_{t-1} + k_t v_t^T.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rule", ["delta", "linear"])
def test_gdn_scalar_gate_page_form(rule):
    rng = np.random.default_rng(41)
    B, T, H, dk, dv = 1, 12, 2, 5, 3
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv)
    a = np.exp(-np.logaddexp(0, rng.standard_normal((B, T, H))) * 0.5)   # [B,T,H]
    o, ST = oracle.kda_forward(q, k, v, a, beta, S0, gate="head", rule=rule)
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            kt, vt, qt, bt, at = k[0, t, h], v[0, t, h], q[0, t, h], beta[0, t, h], a[0, t, h]
            erase = np.eye(dk) - (bt * np.outer(kt, kt) if rule == "delta" else 0.0)
            S = at * (erase @ S) + bt * np.outer(kt, vt)
            assert _rel(o[0, t, h], S.T @ qt) < 1e-12
        assert _rel(ST[0, h], S) < 1e-12


def test_gate_none_is_the_plain_delta_rule():
    rng = np.random.default_rng(42)
    dk, dv, T = 6, 4, 30
    q, k, v, _, beta, S0 = _rand_inputs(rng, 1, T, 1, dk, dv)
    o, ST = oracle.kda_forward(q, k, v, None, beta, S0, gate="none")
    S = S0[0, 0].copy()
    for t in range(T):
        kt, vt, qt, bt = k[0, t, 0], v[0, t, 0], q[0, t, 0], beta[0, t, 0]
        S = S + bt * np.outer(kt, vt - S.T @ kt)        # error form, section 3
        assert _rel(o[0, t, 0], S.T @ qt) < 1e-12
    assert _rel(ST[0, 0], S) < 1e-12


def test_gate_none_linear_beta_one_is_plain_linear_memory():
    rng = np.random.default_rng(43)
    T, dk, dv = 25, 7, 5
    q, k, v, _, _, _ = _rand_inputs(rng, 1, T, 1, dk, dv)
    o, ST = oracle.kda_forward(q, k, v, None, np.ones((1, T, 1)), None, gate="none", rule="linear")
    Q, K, V = q[0, :, 0], k[0, :, 0], v[0, :, 0]
    assert _rel(o[0, :, 0], np.tril(Q @ K.T) @ V) < 1e-13
    assert _rel(ST[0, 0], K.T @ V) < 1e-13


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("rule", ["delta", "linear"])
def test_decode_step_variants_equal_one_token_prefill(gate, rule):
    rng = np.random.default_rng(44)
    B, H, dk, dv = 2, 3, 4, 5
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, B, 1, H, dk, dv)
    a = {"channel": alpha[:, 0], "head": alpha[:, 0, :, 0], "none": None}[gate]
    o1, S1 = oracle.kda_decode_step(q[:, 0], k[:, 0], v[:, 0], a, beta[:, 0], S0, gate=gate, rule=rule)
    # the same step written out per head
    for b in range(B):
        for h in range(H):
            at = {"channel": alpha[b, 0, h], "head": np.full(dk, alpha[b, 0, h, 0]), "none": np.ones(dk)}[gate]
            Sd = at[:, None] * S0[b, h]
            kt, vt, qt, bt = k[b, 0, h], v[b, 0, h], q[b, 0, h], beta[b, 0, h]
            u = bt * (vt - (Sd.T @ kt if rule == "delta" else 0.0))
            Sn = Sd + np.outer(kt, u)
            assert _rel(S1[b, h], Sn) < 1e-13
            assert _rel(o1[b, h], Sn.T @ qt) < 1e-13


# --------------------------------------------------------------------------
# Input prologue (the maps in front of the recurrence): unit q and k per
# (token, head), alpha = exp(-c softplus(g)) in (0, 1], beta = sigmoid(b).
# Pinned by closed forms and by independent library routines.
# --------------------------------------------------------------------------
def test_prologue_unit_vectors_and_zero():
    rng = np.random.default_rng(50)
    q_raw = rng.standard_normal((2, 3, 4, 16)) * 7.0
    k_raw = rng.standard_normal((2, 3, 4, 16))
    k_raw[1, 2, 3] = 0.0
    q, k, _, _ = oracle.input_prologue(q_raw, k_raw, None, np.zeros((2, 3, 4)), 0.1, gate="none")
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=0, atol=1e-14)
    # same direction: q = q_raw / |q_raw| component-wise
    cos = np.sum(q * q_raw, axis=-1) / np.linalg.norm(q_raw, axis=-1)
    assert np.allclose(cos, 1.0, rtol=0, atol=1e-14)
    assert np.all(k[1, 2, 3] == 0.0)
    nz = np.linalg.norm(k, axis=-1)
    nz[1, 2, 3] = 1.0
    assert np.allclose(nz, 1.0, rtol=0, atol=1e-14)


def test_prologue_gate_and_beta_closed_forms():
    c = 0.37
    g = np.array([0.0, 30.0, -30.0, 1.5, -2.25])
    _, _, alpha, beta = oracle.input_prologue(np.ones((5, 2)), np.ones((5, 2)), g, g, c, gate="head")
    assert abs(alpha[0] - 2.0 ** (-c)) < 1e-15                    # softplus(0) = ln 2
    assert abs(np.log(alpha[1]) + c * 30.0) < 1e-12                # softplus(x) -> x
    assert abs(alpha[2] - 1.0) < 1e-12                             # softplus(x) -> 0
    assert abs(beta[0] - 0.5) < 1e-16
    # independent routines: log(1 + e^x) as logaddexp(0, x); the logistic as tanh
    assert np.allclose(alpha, np.exp(-c * np.logaddexp(0.0, g)), rtol=1e-14, atol=0)
    assert np.allclose(beta, 0.5 * (1.0 + np.tanh(0.5 * g)), rtol=1e-14, atol=1e-16)
    assert np.all((alpha > 0) & (alpha <= 1))


def test_prologue_feeds_the_recurrence():
    x = __import__("synth").raw_prefill_inputs(1, 9, 2, 8, 4, dtype="f32", s0_std=0.1, seed=3)
    o1, s1 = oracle.kda_forward_fused(x["q_raw"], x["k_raw"], x["v"], x["g_raw"], x["b_raw"], x["S0"],
                                      gate_scale=0.2)
    q, k, a, b = oracle.input_prologue(x["q_raw"], x["k_raw"], x["g_raw"], x["b_raw"], 0.2)
    o2, s2 = oracle.kda_forward(q, k, x["v"], a, b, x["S0"])
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("rule", ["delta", "linear"])
def test_fused_variants_dense_page_form(gate, rule):
    """The fused oracle for every gate and rule against a loop written from the
    pages with dense matrices, fed by maps computed here from their own
    definitions: unit q and k (section 3's projection reading), alpha =
    exp(-c log(1 + e^g)) as a gate in [0, 1] (section 4), beta the logistic
    function.  The loop applies S_t = A_t S_{t-1} + B_t with A_t =
    (I - beta_t k_t k_t^T) Diag(alpha_t) for the delta rule (section 4) or
    Diag(alpha_t) without the erase (section 2.1's write with the gate), B_t =
    beta_t k_t v_t^T, then reads o_t = S_t^T q_t (section 2.1)."""
    rng = np.random.default_rng(61)
    B, T, H, dk, dv, c = 2, 7, 3, 6, 4, 0.7
    q_raw = rng.standard_normal((B, T, H, dk)) * 3.0
    k_raw = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g_raw = rng.standard_normal((B, T, H, dk) if gate == "channel" else (B, T, H)) * 2.0
    b_raw = rng.standard_normal((B, T, H)) * 2.0
    S0 = 0.2 * rng.standard_normal((B, H, dk, dv))
    o, ST = oracle.kda_forward_fused(q_raw, k_raw, v, None if gate == "none" else g_raw, b_raw, S0,
                                     gate_scale=c, gate=gate, rule=rule)
    for b in range(B):
        for h in range(H):
            S = S0[b, h].copy()
            for t in range(T):
                qv = q_raw[b, t, h] / np.sqrt(q_raw[b, t, h] @ q_raw[b, t, h])
                kv = k_raw[b, t, h] / np.sqrt(k_raw[b, t, h] @ k_raw[b, t, h])
                if gate == "none":
                    a = np.ones(dk)
                else:
                    a = np.broadcast_to(np.exp(-c * np.log1p(np.exp(g_raw[b, t, h]))), (dk,))
                bt = 1.0 / (1.0 + np.exp(-b_raw[b, t, h]))
                A = np.diag(a)
                if rule == "delta":
                    A = (np.eye(dk) - bt * np.outer(kv, kv)) @ A
                S = A @ S + bt * np.outer(kv, v[b, t, h])
                np.testing.assert_allclose(o[b, t, h], S.T @ qv, rtol=0, atol=1e-12)
            np.testing.assert_allclose(ST[b, h], S, rtol=0, atol=1e-12)
