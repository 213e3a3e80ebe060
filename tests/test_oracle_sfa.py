"""Pins of the oracle's sparse feature attention (``oracle.topk_features``, ``oracle.sfa_fwd``).

Scaling Attention via Feature Sparsity, key design 1: Topk_k(x)_u = x_u for u among the k
coordinates of largest |x|, else 0; the scores are the products of the sparsified queries
and keys (nonzero only on shared coordinates), then the usual softmax times V (key design
3: exact, not approximate). Pins: hand examples, including the tie reading (lower index
first); per-row properties (k kept, values unchanged, every kept |x| >= every dropped |x|);
k = d is plain attention (torch SDPA, float64); the scores equal an explicit sum over the
intersection of the two supports; planted mistakes in a copy of the selection fail.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_hand_examples():
    x = np.array([[0.5, -3.0, 2.0, 0.1, -2.0]])
    assert np.array_equal(oracle.topk_features(x, 1), [[0, -3.0, 0, 0, 0]])
    assert np.array_equal(oracle.topk_features(x, 2), [[0, -3.0, 2.0, 0, 0]])   # tie |2|: index 2
    assert np.array_equal(oracle.topk_features(x, 3), [[0, -3.0, 2.0, 0, -2.0]])
    assert np.array_equal(oracle.topk_features(x, 5), x)
    y = np.array([[1.0, 1.0, 1.0, 1.0]])
    assert np.array_equal(oracle.topk_features(y, 2), [[1.0, 1.0, 0, 0]])


@pytest.mark.parametrize("k", [1, 4, 16, 63, 64])
def test_selection_properties(k):
    rng = np.random.default_rng(k)
    X = rng.standard_normal((3, 2, 50, 64))
    X[0, 0, 0] = 0.0                      # an all-zero row
    X[1, 1, 3, :10] = 0.7                 # ties
    T = oracle.topk_features(X, k)
    for r, t in zip(X.reshape(-1, 64), T.reshape(-1, 64)):
        kept = t != 0
        assert kept.sum() <= k and (kept.sum() == k or np.count_nonzero(r) < k)
        assert np.array_equal(t[kept], r[kept])
        if kept.sum() == k and k < 64:
            assert np.abs(r[kept]).min() >= np.abs(r[~kept]).max()


@pytest.mark.parametrize("causal", [False, True])
def test_k_equal_d_is_plain_attention(oracle_mod, causal):
    rng = np.random.default_rng(7 + causal)
    Q, K = rng.standard_normal((1, 2, 40, 16)), rng.standard_normal((1, 2, 40, 16))
    V = rng.standard_normal((1, 2, 40, 8))
    O = oracle.sfa_fwd(Q, K, V, 16, 0.25, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a) for a in (Q, K, V)), is_causal=causal, scale=0.25).numpy()
    assert np.max(np.abs(O - ref)) <= 1e-12


def test_scores_are_support_intersections(oracle_mod):
    rng = np.random.default_rng(9)
    d, k, N = 32, 5, 12
    Q, K = rng.standard_normal((1, 1, N, d)), rng.standard_normal((1, 1, N, d))
    Qs, Ks = oracle.topk_features(Q, k)[0, 0], oracle.topk_features(K, k)[0, 0]
    S = oracle.scores(Qs[None, None], Ks[None, None], np.eye(d)[None], 0.3, False)[0, 0]
    for i in range(N):
        for j in range(N):
            shared = np.flatnonzero((Qs[i] != 0) & (Ks[j] != 0))
            assert abs(S[i, j] - 0.3 * sum(Qs[i, u] * Ks[j, u] for u in shared)) <= 1e-12


def test_planted_selection_mistakes_fail():
    """A copy of the selection with a plausible mistake disagrees with the hand examples."""
    x = np.array([[0.5, -3.0, 2.0, 0.1, -2.0]])

    def by_value(x, k):      # ranks by x instead of |x|
        out = np.zeros_like(x)
        keep = np.argsort(-x[0], kind="stable")[:k]
        out[0, keep] = x[0, keep]
        return out

    def last_tie(x, k):      # ties to the higher index
        out = np.zeros_like(x)
        keep = np.lexsort((-np.arange(5), -np.abs(x[0])))[:k]
        out[0, keep] = x[0, keep]
        return out
    good = oracle.topk_features(x, 2)
    assert not np.array_equal(by_value(x, 2), good)
    assert not np.array_equal(last_tie(x, 2), good)
