"""Pins of the oracle's backward (``oracle.attn_bwd``) to things other than itself.

The backward is the chain rule of the forward definition ("Sparse Projection Attention"
page, Sec. 3.1.3 and Algorithm 1 for the forward; Sec. 3.4.1 Gradient Flow gives the
projection's gradient, Algorithm 2 trains the projection with it). Pins:

* central finite differences of the forward oracle, in double, for every input element of
  tiny problems (queries, keys, values and the projection, both masks, several batches so
  the projection's gradient sums over them);
* float64 autograd through an independent torch formulation of the forward;
* with P = I (m = d), torch's own float64 scaled-dot-product-attention backward;
* closed forms: dO = 0 gives zero gradients; the value gradient is A^T dO with A the
  explicit row softmax; constant V makes O independent of the scores, so the query, key and
  projection gradients vanish; causal row 0 (one key) gives its query no gradient;
* planted mistakes in a copy of the oracle's backward fail the autograd pin.
"""
import contextlib
import ctypes
import math
import os

import numpy as np
import pytest
import torch

import oracle

SHAPES = [  # B, H, N, d, m, dv
    (1, 1, 1, 3, 2, 2),
    (1, 2, 5, 4, 3, 3),
    (2, 1, 7, 3, 5, 2),
]


def _draw(rng, B, H, N, d, m, dv):
    Q, K = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
    V, P = rng.standard_normal((B, H, N, dv)), rng.standard_normal((H, d, m)) / math.sqrt(m)
    dO = rng.standard_normal((B, H, N, dv))
    return Q, K, V, P, dO


def _loss(Q, K, V, P, dO, scale, causal):
    return float(np.sum(dO * oracle.attn_fwd(Q, K, V, P, scale, causal, nthreads=1)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_backward_matches_central_differences(oracle_mod, shape, causal):
    rng = np.random.default_rng(hash((shape, causal)) % (2 ** 32))
    Q, K, V, P, dO = _draw(rng, *shape)
    scale = 0.7
    grads = oracle.attn_bwd(Q, K, V, P, dO, scale, causal, nthreads=1)
    h = 1e-5
    for x, g in zip((Q, K, V, P), grads):
        fd = np.empty_like(x)
        flat = x.reshape(-1)
        for e in range(flat.size):
            keep = flat[e]
            flat[e] = keep + h
            lp = _loss(Q, K, V, P, dO, scale, causal)
            flat[e] = keep - h
            lm = _loss(Q, K, V, P, dO, scale, causal)
            flat[e] = keep
            fd.reshape(-1)[e] = (lp - lm) / (2 * h)
        assert np.max(np.abs(fd - g)) <= 1e-7 * (1.0 + np.max(np.abs(g))), (x.shape, fd, g)


def _torch_grads(Q, K, V, P, dO, scale, causal):
    """float64 autograd through an independent torch formulation of the forward."""
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V, P)]
    Qt = torch.einsum("bhnd,hdm->bhnm", t[0], t[3])
    Kt = torch.einsum("bhnd,hdm->bhnm", t[1], t[3])
    S = scale * torch.matmul(Qt, Kt.transpose(-1, -2))
    if causal:
        N = S.shape[-1]
        S = S.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    O = torch.matmul(torch.softmax(S, dim=-1), t[2])
    (O * torch.from_numpy(dO)).sum().backward()
    return [a.grad.numpy() for a in t]


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_float64_autograd(oracle_mod, causal):
    rng = np.random.default_rng(7 + causal)
    B, H, N, d, m, dv = 2, 3, 70, 16, 8, 12
    Q, K, V, P, dO = _draw(rng, B, H, N, d, m, dv)
    scale = 1.0 / math.sqrt(d)
    ours = oracle.attn_bwd(Q, K, V, P, dO, scale, causal)
    ref = _torch_grads(Q, K, V, P, dO, scale, causal)
    for name, a, b in zip(("dQ", "dK", "dV", "dP"), ours, ref):
        assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(b)), name


@pytest.mark.parametrize("causal", [False, True])
def test_identity_projection_matches_sdpa_backward(oracle_mod, causal):
    rng = np.random.default_rng(11 + causal)
    B, H, N, d, dv = 1, 2, 40, 8, 8
    Q, K, V, _, dO = _draw(rng, B, H, N, d, d, dv)
    P = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    scale = 1.0 / math.sqrt(d)
    dQ, dK, dV, _ = oracle.attn_bwd(Q, K, V, P, dO, scale, causal)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V)]
    O = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=scale)
    (O * torch.from_numpy(dO)).sum().backward()
    for a, b in zip((dQ, dK, dV), t):
        ref = b.grad.numpy()
        assert np.max(np.abs(a - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_closed_forms(oracle_mod):
    rng = np.random.default_rng(3)
    B, H, N, d, m, dv = 1, 2, 9, 5, 4, 3
    Q, K, V, P, dO = _draw(rng, B, H, N, d, m, dv)
    scale = 0.4
    for causal in (False, True):
        # dO = 0: every gradient vanishes
        z = oracle.attn_bwd(Q, K, V, P, np.zeros_like(dO), scale, causal)
        assert all(np.all(g == 0.0) for g in z)
        # dV = A^T dO with A the explicit row softmax
        _, _, dV, _ = oracle.attn_bwd(Q, K, V, P, dO, scale, causal)
        for h in range(H):
            S = scale * (Q[0, h] @ P[h]) @ (K[0, h] @ P[h]).T
            if causal:
                S[np.triu(np.ones((N, N), dtype=bool), 1)] = -np.inf
            A = np.exp(S - S.max(axis=1, keepdims=True))
            A /= A.sum(axis=1, keepdims=True)
            assert np.allclose(dV[0, h], A.T @ dO[0, h], rtol=0, atol=1e-13)
        # V = const makes O independent of the scores: dQ = dK = dP = 0
        g = oracle.attn_bwd(Q, K, np.ones_like(V), P, dO, scale, causal)
        assert max(np.max(np.abs(g[0])), np.max(np.abs(g[1])), np.max(np.abs(g[3]))) <= 1e-13
    # causal row 0 sees only key 0: its query gets no gradient
    dQ, _, _, _ = oracle.attn_bwd(Q, K, V, P, dO, scale, True)
    assert np.all(np.abs(dQ[:, :, 0]) <= 1e-15)


BWD_MUTANTS = {
    "D_i dropped from dS": ("const double dS = a[j] * (dA - Di);", "const double dS = a[j] * dA;"),
    "key gradient from the keys": ("dKt[j * m + c] += scale * dS * Qt[i * m + c];",
                                   "dKt[j * m + c] += scale * dS * Kt[i * m + c];"),
    "value gradient with the row's own weight index": (
        "dVh[j * dv + c] += a[j] * dOh[i * dv + c];", "dVh[j * dv + c] += a[i < nk ? i : j] * dOh[i * dv + c];"),
    "projection gradient without the key term": (
        "dPb[k * m + c] += Qh[n * d + k] * dQt[n * m + c] + Kh[n * d + k] * dKt[n * m + c];",
        "dPb[k * m + c] += Qh[n * d + k] * dQt[n * m + c];"),
    "query gradient without the scale": ("dQt[i * m + c] += scale * dS * Kt[j * m + c];",
                                         "dQt[i * m + c] += dS * Kt[j * m + c];"),
}


@contextlib.contextmanager
def _mutant(tmp_path, old, new):
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, old
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = oracle.build(path, os.path.join(tmp_path, "libmutant.so"))
    saved = oracle._lib
    oracle._lib = oracle.configure(ctypes.CDLL(so))
    try:
        yield
    finally:
        oracle._lib = saved


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_planted_backward_mistake_is_caught(oracle_mod, tmp_path, name):
    old, new = BWD_MUTANTS[name]
    rng = np.random.default_rng(5)
    B, H, N, d, m, dv = 2, 2, 12, 6, 4, 5
    Q, K, V, P, dO = _draw(rng, B, H, N, d, m, dv)
    ref = _torch_grads(Q, K, V, P, dO, 0.5, True)
    with _mutant(str(tmp_path), old, new):
        got = oracle.attn_bwd(Q, K, V, P, dO, 0.5, True)
    assert any(np.max(np.abs(a - b)) > 1e-6 * np.max(np.abs(b)) for a, b in zip(got, ref))
