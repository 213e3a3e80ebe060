"""The oracle's pins have teeth: each planted mistake in a copy of the oracle fails a pin.

Every mutant is a one-line textual change to a temporary copy of ``oracle/spa_oracle.c``,
compiled with gcc on the CPU; the committed oracle is never touched. Each mutant must be
caught by the closed forms and library comparisons the pin suite uses.
"""
import contextlib
import ctypes
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

MUTANTS = {
    "dropped score scale": ("w[j] = scale * acc;", "w[j] = acc;"),
    "diagonal left out of the causal set": (
        "return causal ? i + 1 : N;", "return causal ? (i > 0 ? i : 1) : N;"),
    "transposed projection index": ("acc += x[k] * ph[k * m + c];",
                                    "acc += x[k] * ph[c * d + k];"),
    "weights not normalised": ("const double a = w[j] / sum;", "const double a = w[j];"),
    "values taken in reverse order": ("const double* vj = V + j * dv;",
                                      "const double* vj = V + (nkeys - 1 - j) * dv;"),
    "every head uses head 0's projection": ("const int64_t h = (r / N) % H;",
                                            "const int64_t h = 0;"),
    "reversed feature index in the score": ("acc += qt[c] * Kt[j * m + c];",
                                            "acc += qt[c] * Kt[j * m + (m - 1 - c)];"),
    "exponent sign flipped": ("w[j] = exp(w[j] - mx);", "w[j] = exp(mx - w[j]);"),
}


@contextlib.contextmanager
def _mutant_oracle(tmp_path, old, new):
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


def _pins_hold() -> bool:
    """A compact run of the pin suite's checks; False as soon as one fails."""
    rng = np.random.default_rng(99)
    for causal in (False, True):
        for (B, H, N, d, m, dv) in ((1, 2, 17, 8, 4, 5), (2, 2, 33, 16, 16, 8)):
            Q, K = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
            V, P = rng.standard_normal((B, H, N, dv)), rng.standard_normal((H, d, m))
            scale = 1.0 / math.sqrt(d)
            O = oracle.attn_fwd(Q, K, V, P, scale, causal)
            ref = np.empty_like(O)
            for b in range(B):
                for h in range(H):
                    S = scale * (Q[b, h] @ P[h]) @ (K[b, h] @ P[h]).T
                    if causal:
                        S[np.triu(np.ones((N, N), dtype=bool), k=1)] = -np.inf
                    ref[b, h] = scipy.special.softmax(S, axis=-1) @ V[b, h]
            if not np.max(np.abs(O - ref)) <= 1e-12 * np.max(np.abs(ref)):
                return False
            eye = np.broadcast_to(np.eye(d), (H, d, d)).copy()
            Oi = oracle.attn_fwd(Q, K, V, eye, scale, causal)
            sd = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V),
                is_causal=causal, scale=scale).numpy()
            if not np.max(np.abs(Oi - sd)) <= 1e-12 * np.max(np.abs(sd)):
                return False
    return True


def test_unmutated_oracle_passes(oracle_mod):
    assert _pins_hold()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(oracle_mod, tmp_path, name):
    old, new = MUTANTS[name]
    with np.errstate(all="ignore"), _mutant_oracle(str(tmp_path), old, new):
        caught = not _pins_hold()
    assert caught, f"pins missed the planted mistake: {name}"
