"""Seeded random-shape sweep of the forward, the backward and decode against the oracle
(MI355X only).

120 cases drawn once from a fixed generator (the same list on every run): batch 1-2, heads
1-3, ragged N up to 1200; on the bf16 path d, dv in {64, 128} and m from 8 to 128, on the
fp32 path d up to 256, dv up to 128 and m from 1; both masks; decode with 1-40 queries
against a cache longer than the keys it reads. Tolerances as in the dedicated tests: bf16
max-abs 2e-2 (forward, decode, lse) or 2e-2 of the largest gradient entry per tensor; fp32
1e-4 relative.
"""
import sys

import numpy as np
import pytest
import torch

import jl_feature_projected_amd as spa
import oracle
from jl_feature_projected_amd import inputs

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu-sweep] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a ROCm GPU"
    spa.lib()
    return torch.device("cuda:0")


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = str(rng.choice(["fwd", "fwd", "bwd", "dec"]))
        f32 = bool(rng.random() < 0.25) and kind != "dec"
        B, H, N = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 1201))
        if f32:
            d, dv = int(rng.integers(1, 257)), int(rng.integers(1, 129))
        else:
            d, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
        m = int(rng.integers(1 if f32 else 8, 129))
        causal = bool(rng.integers(0, 2))
        nq = int(rng.integers(1, min(N, 40) + 1))
        extra = int(rng.integers(0, 100))
        out.append((i, kind, B, H, N, d, m, dv, causal, "f32" if f32 else "bf16", nq, extra))
    return out


CASES = _cases(120, 20261203)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_sweep(dev, oracle_mod, case):
    i, kind, B, H, N, d, m, dv, causal, dt, nq, extra = case
    w = inputs.Workload(f"sweep{i}", B, H, N, d, m, dv, causal, dtype=dt, seed=91000 + i)
    x = inputs.draw(w)
    note(f"{case}")
    Q, K, V, P = (t.to(dev) for t in (x.Q, x.K, x.V, x.P))
    if kind == "fwd":
        O, lse = spa.spa_attn_fwd(Q, K, V, P, w.scale, causal, return_lse=True)
        torch.cuda.synchronize()
        Or, lr = oracle.attn_fwd(x.Q, x.K, x.V, x.P, w.scale, causal, with_lse=True)
        if dt == "f32":
            assert rel(np64(O), Or) <= 1e-4
            assert np.max(np.abs(np64(lse) - lr)) <= 1e-4 * max(1.0, np.max(np.abs(lr)))
        else:
            assert np.max(np.abs(np64(O) - Or)) <= 2e-2
            assert np.max(np.abs(np64(lse) - lr)) <= 2e-2
    elif kind == "bwd":
        odt = torch.float32 if dt == "f32" else torch.bfloat16
        O, lse = spa.spa_attn_fwd(Q, K, V, P, w.scale, causal, out_dtype=odt, return_lse=True)
        dO = inputs.draw_grad_output(w, 92000 + i)
        g = spa.spa_attn_bwd(Q, K, V, P, O, dO.to(dev), lse, w.scale, causal)
        torch.cuda.synchronize()
        ref = oracle.attn_bwd(x.Q, x.K, x.V, x.P, dO, w.scale, causal)
        for name, a, r in zip(("dQ", "dK", "dV", "dP"), g, ref):
            assert np.all(np.isfinite(np64(a))), name
            assert rel(np64(a), r) <= (1e-4 if dt == "f32" else 2e-2), name
    else:
        rows = N + extra
        cache = torch.zeros((B, H, rows, m), dtype=torch.float16, device=dev)
        spa.spa_kcache_append(K, P, cache, 0)
        Vc = torch.zeros((B, H, rows, dv), dtype=torch.bfloat16, device=dev)
        Vc[:, :, :N] = V
        Qd = x.Q[:, :, N - nq:].contiguous().to(dev)
        O, lse = spa.spa_attn_decode(Qd, cache, Vc, P, N, w.scale, causal, return_lse=True)
        torch.cuda.synchronize()
        Or, lr = oracle.attn_decode(x.Q[:, :, N - nq:], x.K, x.V, x.P, w.scale, causal,
                                    with_lse=True)
        assert np.max(np.abs(np64(O) - Or)) <= 2e-2
        assert np.max(np.abs(np64(lse) - lr)) <= 2e-2
