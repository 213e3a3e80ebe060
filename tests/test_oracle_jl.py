"""Statistical and deterministic pins of the oracle's projected scores (no GPU).

* Projection-Decomposition Attention (PDA) page, first part Theorem 3.3 (the same statement
  as the revised proof's Theorem 4.1): if m >= 8 d / eps^2 * ln(2 L^2 / delta) then
  max_ij |St_ij - S_ij| <= eps with probability >= 1 - delta, where S = Q K^T / sqrt(d) and
  St = (Q P)(K P)^T / sqrt(d) with P iid N(0, 1/m) (revised proof Sec. 2.1 definition).
* PDA Theorem 3.1 (inner-product JL tail): P(|St_ij - S_ij| >= eps) <= 4 exp(-m eps^2/(8 d))
  for rows of norm sqrt(d), eps/sqrt(d) in (0, 1/2).
* The first two moments of St over P, derived from the N(0, 1/m) definition:
  E[St_ij] = S_ij and Var[St_ij] = (|Q_i|^2 |K_j|^2 / d + S_ij^2) / m.
* PDA Sec. 5.2 / revised Sec. 7 experiment item 1: max |St - S| decays like m^(-1/2).
* Deterministic: PDA revised Lemma 3.2 |softmax(x) - softmax(y)|_1 <= 2 |x - y|_inf; PDA
  revised Theorem 3.4 in the form |o_i - ot_i|_2 <= |a_i - at_i|_1 max_j |v_j|_2; Sparse
  Projection Attention page Lemma 2 |softmax(A) - softmax(B)|_F <= |A - B|_F.
"""
import math

import numpy as np
import pytest

from jl_feature_projected_amd import inputs

SEEDS = 300


def _unit_rows(rng, n, d, corr=0.0):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True) * math.sqrt(d)


def _qk(seed, L, d):
    """Q, K with rows of norm sqrt(d); half of the keys correlate with a query (large S)."""
    rng = np.random.default_rng(seed)
    Q = _unit_rows(rng, L, d)
    K = _unit_rows(rng, L, d)
    K[: L // 2] = Q[: L // 2] + 0.5 * K[: L // 2]
    K = K / np.linalg.norm(K, axis=-1, keepdims=True) * math.sqrt(d)
    return Q[None, None], K[None, None]


def _projected_scores(oracle_mod, Q, K, m, seed):
    d = Q.shape[-1]
    P = inputs.gaussian_projection(d, m, seed)
    return oracle_mod.scores(Q, K, P, 1.0 / math.sqrt(d), False, nthreads=1)[0, 0]


def _exact_scores(Q, K):
    return (Q[0, 0] @ K[0, 0].T) / math.sqrt(Q.shape[-1])


@pytest.mark.parametrize("m", [64, 256, 1024])
def test_theorem_3_3_global_projection_error(oracle_mod, m):
    L, d = 32, 64
    Q, K = _qk(1, L, d)
    S = _exact_scores(Q, K)
    errs = np.array([np.max(np.abs(_projected_scores(oracle_mod, Q, K, m, s) - S))
                     for s in range(SEEDS)])
    for delta in (0.05, 0.2):
        eps = math.sqrt(8.0 * d * math.log(2.0 * L * L / delta) / m)
        frac = np.mean(errs > eps)
        assert frac <= delta + 3.0 * math.sqrt(delta * (1 - delta) / SEEDS), (m, delta, eps)


def test_theorem_3_1_pairwise_tail(oracle_mod):
    L, d, m = 24, 64, 256
    Q, K = _qk(2, L, d)
    S = _exact_scores(Q, K)
    diffs = np.stack([_projected_scores(oracle_mod, Q, K, m, s) - S for s in range(SEEDS)])
    n = diffs.size
    for eps0 in (0.1, 0.2, 0.3, 0.45):  # eps / sqrt(d) inside (0, 1/2)
        eps = eps0 * math.sqrt(d)
        bound = min(1.0, 4.0 * math.exp(-m * eps * eps / (8.0 * d)))
        frac = np.mean(np.abs(diffs) >= eps)
        assert frac <= bound + 3.0 * math.sqrt(max(bound * (1 - bound), 1e-12) / n)


def test_projected_score_moments(oracle_mod):
    """Unbiased, with the closed-form variance, over seeds of P."""
    L, d, m = 12, 32, 8
    Q, K = _qk(3, L, d)
    S = _exact_scores(Q, K)
    St = np.stack([_projected_scores(oracle_mod, Q, K, m, 10_000 + s) for s in range(4 * SEEDS)])
    n = St.shape[0]
    qn = np.sum(Q[0, 0] ** 2, axis=-1)
    kn = np.sum(K[0, 0] ** 2, axis=-1)
    var = (np.outer(qn, kn) / d + S * S) / m
    mean_err = (St.mean(axis=0) - S) / np.sqrt(var / n)
    assert np.max(np.abs(mean_err)) < 5.0
    ratio = St.var(axis=0, ddof=1) / var
    assert 0.93 < np.mean(ratio) < 1.07
    assert 0.6 < np.min(ratio) and np.max(ratio) < 1.5


def test_max_error_decays_like_inverse_sqrt_m(oracle_mod):
    L, d = 32, 64
    Q, K = _qk(4, L, d)
    S = _exact_scores(Q, K)
    ms = np.array([16, 64, 256, 1024])
    med = [np.median([np.max(np.abs(_projected_scores(oracle_mod, Q, K, int(m), s) - S))
                      for s in range(60)]) for m in ms]
    slope = np.polyfit(np.log(ms), np.log(med), 1)[0]
    assert -0.65 <= slope <= -0.40, (slope, med)


def _softmax_rows(x):
    z = x - np.max(x, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_lipschitz_and_output_bounds(oracle_mod, causal):
    L, d, dv = 40, 32, 16
    rng = np.random.default_rng(5)
    Q, K = _qk(5, L, d)
    V = rng.standard_normal((1, 1, L, dv))
    scale = 1.0 / math.sqrt(d)
    eye = np.eye(d)[None]
    A = oracle_mod.weights(Q, K, eye, scale, causal)[0, 0]
    O = oracle_mod.attn_fwd(Q, K, V, eye, scale, causal)[0, 0]
    S = oracle_mod.scores(Q, K, eye, scale, causal)[0, 0]
    vmax = np.max(np.linalg.norm(V[0, 0], axis=-1))
    for seed in range(40):
        for m in (4, 16, 64):
            P = inputs.gaussian_projection(d, m, 500 + seed)
            St = oracle_mod.scores(Q, K, P, scale, causal)[0, 0]
            At = oracle_mod.weights(Q, K, P, scale, causal)[0, 0]
            Ot = oracle_mod.attn_fwd(Q, K, V, P, scale, causal)[0, 0]
            fin = np.isfinite(S)
            dS = np.where(fin, S - np.where(fin, St, 0.0), 0.0)
            l1 = np.sum(np.abs(A - At), axis=-1)
            # revised Lemma 3.2, row by row
            assert np.all(l1 <= 2.0 * np.max(np.abs(dS), axis=-1) + 1e-12)
            # revised Theorem 3.4 (row output), with max_j |v_j| in place of |V|_2
            assert np.all(np.linalg.norm(O - Ot, axis=-1) <= l1 * vmax + 1e-12)
            # SPA Lemma 2 (Frobenius Lipschitz), over the unmasked entries
            assert np.linalg.norm(A - At) <= np.linalg.norm(dS) + 1e-12
    # the oracle's weights are the softmax of its scores on the unmasked set
    if not causal:
        assert np.max(np.abs(A - _softmax_rows(S))) <= 1e-14
