"""Pins of the oracle's rectangular (decode) attention, ``oracle.attn_decode`` (no GPU).

The operation is the forward of the Sparse Projection Attention page (Sec. 3.1.3, Algorithm
1) with fewer queries than keys; the causal mask is aligned to the end of the key sequence
(query i of Nq at position Nk - Nq + i), a reading recorded in the oracle's docstring.
Pins: an explicit numpy softmax over a rectangular mask written out independently; Nq = Nk
equals the square forward; the last query under the causal mask sees every key, so it
equals the unmasked result; a hand example with one query and two keys.
"""
import math

import numpy as np
import pytest

import oracle


def _brute(Q, K, V, P, scale, causal):
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    O = np.empty((B, H, Nq, V.shape[3]))
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            S = scale * (Q[b, h] @ P[h]) @ (K[b, h] @ P[h]).T
            if causal:
                i = np.arange(Nq)[:, None]
                j = np.arange(Nk)[None, :]
                S = np.where(j <= Nk - Nq + i, S, -np.inf)
            mx = S.max(axis=1, keepdims=True)
            E = np.exp(S - mx)
            O[b, h] = (E / E.sum(axis=1, keepdims=True)) @ V[b, h]
            L[b, h] = mx[:, 0] + np.log(E.sum(axis=1))
    return O, L


CASES = [(1, 1, 1, 1, 4, 3, 2), (1, 2, 1, 9, 5, 4, 3), (2, 1, 3, 7, 6, 2, 4),
         (1, 2, 5, 5, 8, 8, 3), (1, 1, 4, 40, 16, 5, 8)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", CASES)
def test_matches_explicit_rectangular_softmax(oracle_mod, shape, causal):
    B, H, Nq, Nk, d, m, dv = shape
    rng = np.random.default_rng(hash(shape) % 2 ** 32)
    Q = rng.standard_normal((B, H, Nq, d))
    K = rng.standard_normal((B, H, Nk, d))
    V = rng.standard_normal((B, H, Nk, dv))
    P = rng.standard_normal((H, d, m)) / math.sqrt(m)
    O, L = oracle.attn_decode(Q, K, V, P, 0.6, causal, with_lse=True)
    Ob, Lb = _brute(Q, K, V, P, 0.6, causal)
    assert np.max(np.abs(O - Ob)) <= 1e-12 * max(1.0, np.max(np.abs(Ob)))
    assert np.max(np.abs(L - Lb)) <= 1e-12 * max(1.0, np.max(np.abs(Lb)))


@pytest.mark.parametrize("causal", [False, True])
def test_square_case_is_the_forward(oracle_mod, causal):
    rng = np.random.default_rng(3)
    Q, K = rng.standard_normal((2, 2, 33, 16)), rng.standard_normal((2, 2, 33, 16))
    V, P = rng.standard_normal((2, 2, 33, 8)), rng.standard_normal((2, 16, 4)) / 2.0
    a = oracle.attn_decode(Q, K, V, P, 0.25, causal)
    b = oracle.attn_fwd(Q, K, V, P, 0.25, causal)
    assert np.max(np.abs(a - b)) <= 1e-13


def test_last_query_sees_every_key(oracle_mod):
    rng = np.random.default_rng(4)
    Q, K = rng.standard_normal((1, 3, 1, 32)), rng.standard_normal((1, 3, 50, 32))
    V, P = rng.standard_normal((1, 3, 50, 16)), rng.standard_normal((3, 32, 8)) / math.sqrt(8)
    a = oracle.attn_decode(Q, K, V, P, 0.2, True)
    b = oracle.attn_decode(Q, K, V, P, 0.2, False)
    assert np.array_equal(a, b)


def test_hand_example(oracle_mod):
    # one query, two keys, P = I (d = m = 1), scale 1: scores 0 and ln 3 -> weights 1/4, 3/4
    Q = np.array([[[[1.0]]]])
    K = np.array([[[[0.0], [math.log(3.0)]]]])
    V = np.array([[[[4.0], [8.0]]]])
    P = np.array([[[1.0]]])
    O = oracle.attn_decode(Q, K, V, P, 1.0, True)
    assert abs(O[0, 0, 0, 0] - (0.25 * 4.0 + 0.75 * 8.0)) <= 1e-14
