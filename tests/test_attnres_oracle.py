"""Pins for the AttnRes oracle (page "Yanjiu KimiK3 ...", section 8): the
weights are a softmax over the earlier layers and the output is their
weighted sum.  Each check is fixed by mathematics, not by the oracle's own
formula."""
import numpy as np
import pytest

from oracle.attnres import attnres_forward


def _rand(rng, L, N, dk, d):
    return rng.standard_normal((N, dk)), rng.standard_normal((L, N, dk)), rng.standard_normal((L, N, d))


def test_single_layer_is_identity():
    rng = np.random.default_rng(0)
    q, k, h = _rand(rng, 1, 5, 8, 6)
    assert np.array_equal(attnres_forward(q, k, h), h[0])


def test_equal_keys_give_the_plain_average():
    rng = np.random.default_rng(1)
    q, k, h = _rand(rng, 7, 4, 8, 5)
    k[:] = k[0]                                      # every layer the same key
    assert np.allclose(attnres_forward(q, k, h), h.mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_layer_is_selected():
    rng = np.random.default_rng(2)
    L, N, dk, d = 9, 3, 4, 6
    q, k, h = _rand(rng, L, N, dk, d)
    k[:] = 0.0
    for n in range(N):
        j = (3 * n + 1) % L
        k[j, n] = 200.0 * q[n] / np.dot(q[n], q[n])  # score 200 for layer j, 0 for the rest
        out = attnres_forward(q[n:n + 1], k[:, n:n + 1], h[:, n:n + 1])
        assert np.allclose(out[0], h[j, n], rtol=0, atol=1e-70)


def test_two_layers_closed_form():
    rng = np.random.default_rng(3)
    q, k, h = _rand(rng, 2, 6, 5, 4)
    s0, s1 = np.sum(q * k[0], axis=1), np.sum(q * k[1], axis=1)
    w1 = 1.0 / (1.0 + np.exp(s0 - s1))               # logistic of the score gap
    expect = (1.0 - w1)[:, None] * h[0] + w1[:, None] * h[1]
    assert np.allclose(attnres_forward(q, k, h), expect, rtol=1e-13, atol=1e-15)


def test_layer_order_does_not_matter():
    rng = np.random.default_rng(4)
    q, k, h = _rand(rng, 11, 5, 6, 7)
    perm = rng.permutation(11)
    assert np.allclose(attnres_forward(q, k, h), attnres_forward(q, k[perm], h[perm]), rtol=1e-13, atol=1e-15)


def test_convex_combination_bounds_and_shift_invariance():
    rng = np.random.default_rng(5)
    q, k, h = _rand(rng, 6, 8, 4, 3)
    out = attnres_forward(q, k, h)
    assert np.all(out <= h.max(axis=0) + 1e-12) and np.all(out >= h.min(axis=0) - 1e-12)
    # adding the same vector to every key shifts every score of a token equally
    shift = rng.standard_normal(4)
    assert np.allclose(attnres_forward(q, k + shift, h), out, rtol=1e-12, atol=1e-14)


def test_large_scores_stay_finite():
    q = np.full((1, 2), 300.0)
    k = np.array([[[1.0, 1.0]], [[1.1, 1.0]]])        # scores 600 and 630
    h = np.array([[[1.0]], [[2.0]]])
    out = attnres_forward(q, k, h)
    assert np.isfinite(out).all()
    assert abs(out[0, 0] - (1.0 + 1.0 / (1.0 + np.exp(-30.0)))) < 1e-12


def test_shape_errors():
    with pytest.raises(ValueError):
        attnres_forward(np.zeros((2, 3)), np.zeros((4, 2, 5)), np.zeros((4, 2, 6)))
