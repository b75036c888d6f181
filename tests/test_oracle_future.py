"""Pins for the future-query importance oracle (CPU only).

Future Forcing summary page, "Componenti Algorithmiche", module 1: keys are scored by their predicted
attention weight under proxy queries. The importance oracle is pinned to the attention oracle (with
identity values the attention output is the weight vector itself), to the pure-loop brute force, and
to properties of softmax weights: each head's importances sum to 1, identical keys share the mass
equally, permuting keys permutes scores, repeating proxies changes nothing.
"""
import numpy as np
import pytest

from oracle import attention as oatt
from oracle import brute
from oracle import future as ofu


def test_single_proxy_equals_attention_weights_via_identity_values():
    rng = np.random.default_rng(0)
    H, n_k = 3, 11
    dh = n_k                                  # value width = key width for the attention oracle
    q = rng.standard_normal((1, H, dh))
    k = rng.standard_normal((n_k, H, dh))
    v = np.broadcast_to(np.eye(n_k)[:, None, :], (n_k, H, n_k)).copy()     # value of key j = e_j
    weights = oatt.attention(q, k, v, 0.6)["A"].reshape(H, n_k)
    np.testing.assert_allclose(ofu.importance(q, k, 0.6), weights, rtol=0, atol=1e-14)


def test_matches_brute_force_loops():
    rng = np.random.default_rng(1)
    H, n_k, n_p = 2, 6, 5
    dh = n_k                                  # value width = key width for the loops
    q = rng.standard_normal((n_p, H, dh))
    k = rng.standard_normal((n_k, H, dh))
    eye = [[[1.0 if c == j else 0.0 for c in range(n_k)] for _ in range(H)] for j in range(n_k)]
    A, _ = brute.attention_loops(q.tolist(), k.tolist(), eye, 0.9)
    want = np.array([[np.mean([A[i][h][j] for i in range(n_p)]) for j in range(n_k)] for h in range(H)])
    np.testing.assert_allclose(ofu.importance(q, k, 0.9), want, rtol=0, atol=1e-14)


def test_softmax_properties():
    rng = np.random.default_rng(2)
    H, dh, n_k, n_p = 2, 16, 40, 9
    q = rng.standard_normal((n_p, H, dh))
    k = rng.standard_normal((n_k, H, dh))
    imp = ofu.importance(q, k, 0.25, block=4)
    np.testing.assert_allclose(imp.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.all(imp > 0)
    perm = rng.permutation(n_k)
    np.testing.assert_allclose(ofu.importance(q, k[perm], 0.25), imp[:, perm], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ofu.importance(np.concatenate([q, q, q]), k, 0.25), imp, rtol=0, atol=1e-14)
    same = np.repeat(k[:1], 7, axis=0)
    np.testing.assert_allclose(ofu.importance(q, same, 0.25), np.full((H, 7), 1.0 / 7), rtol=0, atol=1e-15)


def test_token_and_hybrid_scores():
    imp = np.array([[0.5, 0.25, 0.25], [0.1, 0.2, 0.7]])
    np.testing.assert_allclose(ofu.token_scores(imp), [0.3, 0.225, 0.475], rtol=0, atol=1e-15)
    f, h = np.array([0.2, 0.8]), np.array([0.6, 0.4])
    np.testing.assert_array_equal(ofu.hybrid(f, h, 1.0), f)
    np.testing.assert_array_equal(ofu.hybrid(f, h, 0.0), h)
    np.testing.assert_allclose(ofu.hybrid(f, h, 0.25), [0.5, 0.5], rtol=0, atol=1e-15)


@pytest.mark.parametrize("scale", [0.1, 2.0])
def test_large_scores_stay_finite(scale):
    rng = np.random.default_rng(3)
    q = 30 * rng.standard_normal((4, 1, 8))
    k = 30 * rng.standard_normal((9, 1, 8))
    imp = ofu.importance(q, k, scale)
    assert np.all(np.isfinite(imp))
    np.testing.assert_allclose(imp.sum(axis=1), 1.0, rtol=0, atol=1e-13)
