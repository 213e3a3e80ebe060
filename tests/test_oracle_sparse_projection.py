"""Pins for fixed sparse and structured projections (no GPU).

* Sparse Projection Attention page, Sec. 2.2 Definition 1: entries sqrt(s/m) * {+1, 0, -1}
  with probabilities 1/(2s), 1 - 1/s, 1/(2s). Checked: the value set, the frequencies
  (binomial bounds) and E[P P^T] = I (each entry has variance 1/m).
* Proposition 1 (sparse JL guarantee, via Achlioptas' Theorem 1.1): at s = 3 the sparse
  matrix is Achlioptas' own and carries the Gaussian JL constants, so the PDA Theorem 3.3
  bound (first part; revised Theorem 4.1) holds with the same rates over seeds; at
  s = sqrt(d) (the proposition's s = O(sqrt(d))) the projected scores stay unbiased and the
  max error still decays like m^(-1/2).
* Block and banded patterns (named in the page's Sec. 3.2 and Table 6, not defined there;
  the generators' readings): the zero pattern, E[P P^T] = I, and unbiased projected scores.
The oracle itself is unchanged: these pins use its `scores` on such P.
"""
import math

import numpy as np
import pytest

from jl_feature_projected_amd import inputs

SEEDS = 300


def _qk(seed, L, d):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((L, d))
    K = rng.standard_normal((L, d))
    K[: L // 2] = Q[: L // 2] + 0.5 * K[: L // 2]
    Q *= math.sqrt(d) / np.linalg.norm(Q, axis=-1, keepdims=True)
    K *= math.sqrt(d) / np.linalg.norm(K, axis=-1, keepdims=True)
    return Q[None, None], K[None, None]


def _exact(Q, K):
    return (Q[0, 0] @ K[0, 0].T) / math.sqrt(Q.shape[-1])


def _st(oracle_mod, Q, K, P):
    d = Q.shape[-1]
    return oracle_mod.scores(Q, K, P[None], 1.0 / math.sqrt(d), False, nthreads=1)[0, 0]


@pytest.mark.parametrize("s", [1.0, 3.0, math.sqrt(128), 20.0])
def test_definition_1_entries(s):
    d, m, draws = 128, 32, 200
    rng = np.random.default_rng(int(10 * s))
    P = np.stack([inputs.sparse_projection(rng, d, m, s) for _ in range(draws)])
    a = math.sqrt(s / m)
    vals = np.unique(P)
    assert set(np.round(vals / a, 12)) <= {-1.0, 0.0, 1.0}
    n = P.size
    for v, prob in ((a, 0.5 / s), (-a, 0.5 / s), (0.0, 1.0 - 1.0 / s)):
        k = np.count_nonzero(P == v)
        sd = math.sqrt(n * prob * (1.0 - prob))
        assert abs(k - n * prob) <= 5.0 * sd + 1e-9, (s, v, k, n * prob)
    G = np.einsum("tij,tkj->ik", P, P) / draws  # E[P P^T] estimate
    # each entry of P P^T is a sum of m independent terms; its sd over one draw is at most
    # sqrt(m * E[x^4]) = sqrt(m * s / m^2) on the diagonal
    sd = math.sqrt(s / m / draws) + 1e-12
    assert np.max(np.abs(G - np.eye(d))) <= 6.0 * sd


def _sparse_scores(oracle_mod, Q, K, m, s, seed):
    d = Q.shape[-1]
    P = inputs.sparse_projection(np.random.default_rng(seed), d, m, s)
    return _st(oracle_mod, Q, K, P)


@pytest.mark.parametrize("m", [64, 256])
def test_proposition_1_at_s3_meets_theorem_3_3(oracle_mod, m):
    L, d = 32, 64
    Q, K = _qk(1, L, d)
    S = _exact(Q, K)
    errs = np.array([np.max(np.abs(_sparse_scores(oracle_mod, Q, K, m, 3.0, s) - S))
                     for s in range(SEEDS)])
    for delta in (0.05, 0.2):
        eps = math.sqrt(8.0 * d * math.log(2.0 * L * L / delta) / m)
        frac = np.mean(errs > eps)
        assert frac <= delta + 3.0 * math.sqrt(delta * (1 - delta) / SEEDS), (m, delta)


def test_proposition_1_at_sqrt_d_unbiased_and_decaying(oracle_mod):
    L, d = 16, 64
    s = math.sqrt(d)
    Q, K = _qk(2, L, d)
    S = _exact(Q, K)
    m = 16
    St = np.stack([_sparse_scores(oracle_mod, Q, K, m, s, 5000 + t) for t in range(4 * SEEDS)])
    sd = St.std(axis=0, ddof=1)
    z = (St.mean(axis=0) - S) / (sd / math.sqrt(St.shape[0]))
    assert np.max(np.abs(z)) < 5.0
    ms = np.array([16, 64, 256, 1024])
    med = [np.median([np.max(np.abs(_sparse_scores(oracle_mod, Q, K, int(mm), s, t) - S))
                      for t in range(60)]) for mm in ms]
    slope = np.polyfit(np.log(ms), np.log(med), 1)[0]
    assert -0.65 <= slope <= -0.40, (slope, med)


STRUCTURED = [("block", (16, 4)), ("block", (8, 8)), ("banded", 16), ("banded", 5)]


def _structured(rng, d, m, kind, arg):
    if kind == "block":
        return inputs.block_projection(rng, d, m, *arg)
    return inputs.banded_projection(rng, d, m, arg)


@pytest.mark.parametrize("kind,arg", STRUCTURED)
def test_structured_pattern_and_isotropy(kind, arg):
    d, m, draws = 128, 32, 400
    rng = np.random.default_rng(7)
    P = np.stack([_structured(rng, d, m, kind, arg) for _ in range(draws)])
    nz = P[0] != 0
    per_row = arg[1] if kind == "block" else arg
    assert np.all(nz.sum(axis=1) == per_row)
    assert np.all((P != 0) == nz)  # the pattern is fixed, only the values are random
    if kind == "block":
        a, b = arg
        for i in range(d):
            c = (i // a) % (m // b)
            assert np.array_equal(np.flatnonzero(nz[i]), np.arange(b * c, b * c + b))
    else:
        for i in range(d):
            center = i * m // d
            dist = (np.flatnonzero(nz[i]) - center + m // 2) % m - m // 2
            assert np.all((dist >= -(arg // 2)) & (dist < arg - arg // 2))
    G = np.einsum("tij,tkj->ik", P, P) / draws
    assert np.max(np.abs(np.diag(G) - 1.0)) <= 6.0 * math.sqrt(2.0 / per_row / draws)
    off = G - np.diag(np.diag(G))
    assert np.max(np.abs(off)) <= 6.0 * math.sqrt(1.0 / per_row / draws) + 1e-12


@pytest.mark.parametrize("kind,arg", STRUCTURED)
def test_structured_scores_unbiased(oracle_mod, kind, arg):
    L, d, m = 12, 128, 32
    Q, K = _qk(3, L, d)
    S = _exact(Q, K)
    rng = np.random.default_rng(11)
    St = np.stack([_st(oracle_mod, Q, K, _structured(rng, d, m, kind, arg)) for _ in range(800)])
    z = (St.mean(axis=0) - S) / (St.std(axis=0, ddof=1) / math.sqrt(St.shape[0]))
    assert np.max(np.abs(z)) < 5.0
