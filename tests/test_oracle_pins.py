"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: an explicit N x N brute
force built from numpy/scipy library routines, torch's float64 scaled-dot-product attention
(the exact-attention special case P = I), or a closed form.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

from jl_feature_projected_amd import inputs


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def brute_force(Q, K, V, P, scale, causal):
    """Explicit N x N evaluation: project, score, -inf mask, full-row softmax, times V."""
    B, H, N, _ = Q.shape
    O = np.empty((B, H, N, V.shape[-1]))
    S_all = np.empty((B, H, N, N))
    for b in range(B):
        for h in range(H):
            qt = Q[b, h] @ P[h]
            kt = K[b, h] @ P[h]
            S = scale * (qt @ kt.T)
            if causal:
                S = np.where(np.triu(np.ones((N, N), dtype=bool), k=1), -np.inf, S)
            A = scipy.special.softmax(S, axis=-1)
            O[b, h] = A @ V[b, h]
            S_all[b, h] = S
    return O, S_all


def _rel_err(a, b):
    denom = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / denom


# --- whole path against the explicit N x N brute force on tiny inputs ----------------------

NS = (1, 2, 3, 7, 16, 33, 64, 130)
DS = (1, 4, 8, 64)
MS = (1, 2, 8, 16, 64)
DVS = (1, 5, 64)


@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_brute_force(oracle_mod, causal):
    rng = np.random.default_rng(7 + causal)
    for N, d, m, dv in itertools.product(NS, DS, MS, DVS):
        B, H = (1, 2) if N > 33 else (2, 2)
        Q, K = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
        V, P = _rand(rng, B, H, N, dv), _rand(rng, H, d, m) / math.sqrt(m)
        scale = 1.0 / math.sqrt(d)
        O = oracle_mod.attn_fwd(Q, K, V, P, scale, causal)
        Ob, _ = brute_force(Q, K, V, P, scale, causal)
        assert _rel_err(O, Ob) <= 1e-12, (N, d, m, dv, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_matches_logsumexp(oracle_mod, causal):
    rng = np.random.default_rng(11)
    Q, K, V = _rand(rng, 2, 3, 37, 16), _rand(rng, 2, 3, 37, 16), _rand(rng, 2, 3, 37, 8)
    P = _rand(rng, 3, 16, 8) / math.sqrt(8)
    _, lse = oracle_mod.attn_fwd(Q, K, V, P, 0.25, causal, with_lse=True)
    _, S = brute_force(Q, K, V, P, 0.25, causal)
    ref = scipy.special.logsumexp(S, axis=-1)
    assert np.max(np.abs(lse - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_scores_and_weights_match_brute_force(oracle_mod):
    rng = np.random.default_rng(12)
    for causal in (False, True):
        Q, K, V = _rand(rng, 1, 2, 19, 8), _rand(rng, 1, 2, 19, 8), _rand(rng, 1, 2, 19, 4)
        P = _rand(rng, 2, 8, 3)
        S = oracle_mod.scores(Q, K, P, 0.3, causal)
        _, Sb = brute_force(Q, K, V, P, 0.3, causal)
        fin = np.isfinite(Sb)
        assert np.array_equal(fin, np.isfinite(S))
        assert np.all(S[~fin] == -np.inf)
        assert _rel_err(S[fin], Sb[fin]) <= 1e-13
        A = oracle_mod.weights(Q, K, P, 0.3, causal)
        assert _rel_err(A, scipy.special.softmax(Sb, axis=-1)) <= 1e-13


def test_rows_variant_equals_full(oracle_mod):
    rng = np.random.default_rng(13)
    for causal in (False, True):
        B, H, N, d, m, dv = 2, 3, 50, 16, 4, 7
        Q, K, V = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d), _rand(rng, B, H, N, dv)
        P = _rand(rng, H, d, m)
        O, lse = oracle_mod.attn_fwd(Q, K, V, P, 0.2, causal, with_lse=True)
        bh = rng.integers(0, B * H, size=40)
        ri = rng.integers(0, N, size=40)
        Or, lr = oracle_mod.attn_rows(Q, K, V, P, 0.2, causal, bh, ri, with_lse=True)
        Of, lf = O.reshape(B * H, N, dv), lse.reshape(B * H, N)
        assert np.array_equal(Or, Of[bh, ri])
        assert np.array_equal(lr, lf[bh, ri])


# --- m = d with P = I is exact attention (SPA page Sec. 3.1.1 vs 3.1.3) ------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,dv", [(1, 8, 8), (17, 8, 3), (64, 64, 64), (130, 32, 16)])
def test_identity_projection_is_exact_attention(oracle_mod, causal, N, d, dv):
    rng = np.random.default_rng(N * 1000 + d)
    B, H = 2, 3
    Q, K, V = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d), _rand(rng, B, H, N, dv)
    P = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    scale = 1.0 / math.sqrt(d)
    O = oracle_mod.attn_fwd(Q, K, V, P, scale, causal)
    # projected keys are the keys themselves, bit for bit
    assert np.array_equal(oracle_mod.project(Q, P), Q)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), is_causal=causal,
        scale=scale).numpy()
    assert _rel_err(O, ref) <= 1e-12
    # a separately written naive softmax(Q K^T / sqrt(d)) V
    S = np.einsum("bhid,bhjd->bhij", Q, K) * scale
    if causal:
        S[..., np.triu(np.ones((N, N), dtype=bool), k=1)] = -np.inf
    S = S - S.max(axis=-1, keepdims=True)
    W = np.exp(S)
    W /= W.sum(axis=-1, keepdims=True)
    assert _rel_err(O, W @ V) <= 1e-12


# --- the projection itself --------------------------------------------------------------

def test_project_matches_matmul_and_selectors(oracle_mod):
    rng = np.random.default_rng(21)
    X, P = _rand(rng, 2, 3, 29, 12), _rand(rng, 3, 12, 5)
    ref = np.einsum("bhnd,hdm->bhnm", X, P)
    assert _rel_err(oracle_mod.project(X, P), ref) <= 1e-13
    # column selector: P = I[:, idx] picks coordinates exactly
    idx = [7, 0, 3]
    sel = np.broadcast_to(np.eye(12)[:, idx], (3, 12, 3)).copy()
    assert np.array_equal(oracle_mod.project(X, sel), X[..., idx])


def test_column_selector_projection_is_attention_on_selected_coordinates(oracle_mod):
    rng = np.random.default_rng(22)
    B, H, N, d, dv = 1, 2, 45, 16, 8
    Q, K, V = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d), _rand(rng, B, H, N, dv)
    idx = [1, 4, 9, 15]
    P = np.broadcast_to(np.eye(d)[:, idx], (H, d, len(idx))).copy()
    for causal in (False, True):
        O = oracle_mod.attn_fwd(Q, K, V, P, 0.37, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[..., idx].copy()), torch.from_numpy(K[..., idx].copy()),
            torch.from_numpy(V), is_causal=causal, scale=0.37).numpy()
        assert _rel_err(O, ref) <= 1e-12


# --- closed forms -----------------------------------------------------------------------

def test_zero_queries_give_uniform_weights(oracle_mod):
    rng = np.random.default_rng(31)
    B, H, N, d, m, dv = 1, 2, 40, 8, 4, 6
    Q = np.zeros((B, H, N, d))
    K, V, P = _rand(rng, B, H, N, d), _rand(rng, B, H, N, dv), _rand(rng, H, d, m)
    O = oracle_mod.attn_fwd(Q, K, V, P, 0.5, False)
    assert _rel_err(O, np.broadcast_to(V.mean(axis=2, keepdims=True), O.shape)) <= 1e-13
    # causal: prefix means, a direct test of the mask
    O = oracle_mod.attn_fwd(Q, K, V, P, 0.5, True)
    prefix = np.cumsum(V, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert _rel_err(O, prefix) <= 1e-13
    # scale = 0 gives the same uniform weights whatever the queries
    O0 = oracle_mod.attn_fwd(_rand(rng, B, H, N, d), K, V, P, 0.0, True)
    assert _rel_err(O0, prefix) <= 1e-13


def test_causal_first_row_is_first_value_exactly(oracle_mod):
    rng = np.random.default_rng(32)
    Q, K, V = _rand(rng, 2, 2, 9, 4), _rand(rng, 2, 2, 9, 4), _rand(rng, 2, 2, 9, 5)
    O = oracle_mod.attn_fwd(Q, K, V, _rand(rng, 2, 4, 3), 1.3, True)
    assert np.array_equal(O[:, :, 0], V[:, :, 0])


def test_rows_of_weights_sum_to_one(oracle_mod):
    rng = np.random.default_rng(33)
    for causal in (False, True):
        Q, K = 3 * _rand(rng, 2, 2, 70, 16), 3 * _rand(rng, 2, 2, 70, 16)
        A = oracle_mod.weights(Q, K, _rand(rng, 2, 16, 8), 0.25, causal)
        assert np.max(np.abs(A.sum(axis=-1) - 1.0)) <= 1e-12
        assert np.all(A >= 0.0)
        if causal:
            assert np.all(A[..., np.triu(np.ones((70, 70), dtype=bool), k=1)] == 0.0)
        # constant values pass through unchanged
        V = np.full((2, 2, 70, 3), 1.75)
        O = oracle_mod.attn_fwd(Q, K, V, _rand(rng, 2, 16, 8), 0.25, causal)
        assert np.max(np.abs(O - 1.75)) <= 1e-12


def test_value_identity_exposes_weights(oracle_mod):
    rng = np.random.default_rng(34)
    N = 24
    Q, K = _rand(rng, 1, 1, N, 8), _rand(rng, 1, 1, N, 8)
    P = _rand(rng, 1, 8, 4)
    V = np.eye(N)[None, None]
    for causal in (False, True):
        O = oracle_mod.attn_fwd(Q, K, V, P, 0.4, causal)
        A = oracle_mod.weights(Q, K, P, 0.4, causal)
        assert _rel_err(O, A) <= 1e-13


def test_noncausal_permutation_equivariance_and_linearity(oracle_mod):
    rng = np.random.default_rng(35)
    B, H, N, d, m, dv = 1, 2, 31, 8, 4, 5
    Q, K, V = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d), _rand(rng, B, H, N, dv)
    P = _rand(rng, H, d, m)
    O = oracle_mod.attn_fwd(Q, K, V, P, 0.6, False)
    perm = rng.permutation(N)
    Ok = oracle_mod.attn_fwd(Q, K[:, :, perm], V[:, :, perm], P, 0.6, False)
    assert _rel_err(Ok, O) <= 1e-13
    Oq = oracle_mod.attn_fwd(Q[:, :, perm], K, V, P, 0.6, False)
    assert _rel_err(Oq, O[:, :, perm]) <= 1e-13
    V2 = _rand(rng, B, H, N, dv)
    for causal in (False, True):
        lhs = oracle_mod.attn_fwd(Q, K, 2.0 * V - 3.0 * V2, P, 0.6, causal)
        rhs = (2.0 * oracle_mod.attn_fwd(Q, K, V, P, 0.6, causal)
               - 3.0 * oracle_mod.attn_fwd(Q, K, V2, P, 0.6, causal))
        assert _rel_err(lhs, rhs) <= 1e-12


def test_hand_computed_two_key_example(oracle_mod):
    """N=2, d=2, m=1: scores chosen so the softmax weights are 1/4 and 3/4 in closed form."""
    # P picks coordinate 0; Qt_1 = 1, Kt = (0, ln 3); scale 1 -> row 1 scores (0, ln 3)
    P = np.array([[[1.0], [0.0]]])
    Q = np.array([[[[5.0, 2.0], [1.0, -4.0]]]])
    K = np.array([[[[0.0, 9.0], [math.log(3.0), 1.0]]]])
    V = np.array([[[[8.0, -4.0], [4.0, 12.0]]]])
    O = oracle_mod.attn_fwd(Q, K, V, P, 1.0, False)
    # row 1: weights (1/4, 3/4) -> (0.25*8 + 0.75*4, 0.25*-4 + 0.75*12) = (5, 8)
    assert np.allclose(O[0, 0, 1], [5.0, 8.0], rtol=0, atol=1e-14)
    # row 0: scores (0, 5 ln 3) -> weights (1/244, 243/244)
    w = np.array([1.0, 243.0]) / 244.0
    assert np.allclose(O[0, 0, 0], w @ V[0, 0], rtol=0, atol=1e-13)
    # causal: row 0 sees key 0 only
    Oc = oracle_mod.attn_fwd(Q, K, V, P, 1.0, True)
    assert np.array_equal(Oc[0, 0, 0], V[0, 0, 0])
    assert np.allclose(Oc[0, 0, 1], [5.0, 8.0], rtol=0, atol=1e-14)


def test_bad_arguments_are_rejected(oracle_mod):
    rng = np.random.default_rng(36)
    Q = _rand(rng, 1, 1, 4, 2)
    with pytest.raises(ValueError):
        oracle_mod.attn_fwd(Q, Q, Q, _rand(rng, 1, 2, 2), float("nan"), False)
    with pytest.raises(ValueError):
        oracle_mod.attn_rows(Q, Q, Q, _rand(rng, 1, 2, 2), 1.0, False, [0], [4])


# --- the seeded workloads themselves ----------------------------------------------------

def test_workload_recipe_properties():
    w = inputs.WORKLOADS["c2"].replace(B=1, H=2, N=64)
    x = inputs.draw_f64(w)
    assert np.allclose(np.linalg.norm(x["Q"], axis=-1), math.sqrt(w.d))
    assert np.allclose(np.linalg.norm(x["V"], axis=-1), math.sqrt(w.dv))
    st = inputs.draw(w)
    assert st.Q.dtype == torch.bfloat16 and st.P.shape == (2, 64, 16)
    # stored values are the float64 draws rounded to bf16
    assert np.max(np.abs(st.f64("Q") - x["Q"])) <= 2.0 ** -8 * np.max(np.abs(x["Q"]))
    # low-rank recipe: V left unnormalised, Q/K rows at sqrt(d)
    w3 = inputs.WORKLOADS["c3"].replace(B=1, H=1, N=256)
    x3 = inputs.draw_f64(w3)
    assert np.allclose(np.linalg.norm(x3["K"], axis=-1), math.sqrt(128))
    assert not np.allclose(np.linalg.norm(x3["V"], axis=-1), math.sqrt(128))
    # the rank-16 signal dominates: 16 singular values carry nearly all of the energy
    s = np.linalg.svd(x3["Q"][0, 0], compute_uv=False)
    assert np.sum(s[:16] ** 2) / np.sum(s ** 2) > 0.98
    # deterministic
    assert np.array_equal(inputs.draw(w).K.float().numpy(), st.K.float().numpy())
    # identity projection
    wi = inputs.WORKLOADS["c5_identity"].replace(N=8)
    assert np.array_equal(inputs.draw(wi).P[3].float().numpy(), np.eye(128))
