"""spa_attention (the autograd wrapper over spa_attn_fwd / spa_attn_bwd) on MI355X.

The wrapper only routes calls: its forward must be the library's forward bit for bit, and
loss.backward() must hand Q, K, V and P the gradients spa_attn_bwd computes for dL/dO, which
the oracle's backward pins (same 2e-2-of-the-largest-entry budget as the backward's own
parity tests for bf16; 1e-4 for the fp32 path). The dK and dV of the wrapper equal those of
a direct spa_attn_bwd call bit for bit; dQ and dP are compared within rounding, since at
m <= 64 the projected-query gradient is summed by atomic adds in a run-dependent order.
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
    print(f"[gpu-autograd] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a ROCm GPU"
    spa.lib()
    return torch.device("cuda:0")


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def close(name, got, ref, tol):
    err, top = np.max(np.abs(got - ref)), np.max(np.abs(ref))
    note(f"{name}: max-abs {err:.3e} of max {top:.3e}")
    assert np.all(np.isfinite(got)), name
    assert err <= tol * top, name


CASES = [  # B, H, N, d, m, dv, causal, dtype
    (2, 2, 300, 128, 32, 128, True, "bf16"),
    (1, 3, 257, 64, 16, 64, False, "bf16"),
    (2, 1, 200, 128, 128, 128, True, "bf16"),
    (1, 2, 130, 64, 16, 64, True, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_autograd_matches_library_and_oracle(dev, oracle_mod, case):
    B, H, N, d, m, dv, causal, dt = case
    note(f"case {case}")
    w = inputs.Workload(f"autograd-{N}", B, H, N, d, m, dv, causal, dtype=dt, seed=3100 + N)
    x = inputs.draw(w)
    G = inputs.draw_grad_output(w, seed=3200 + N)
    leaves = [t.to(dev).requires_grad_(True) for t in (x.Q, x.K, x.V, x.P)]
    Q, K, V, P = leaves
    O = spa.spa_attention(Q, K, V, P, w.scale, causal)
    Gd = G.to(dev)
    (O.float() * Gd.float()).sum().backward()
    torch.cuda.synchronize()

    # the wrapper's forward is the library's forward
    with torch.no_grad():
        O_lib, lse = spa.spa_attn_fwd(Q.detach(), K.detach(), V.detach(), P.detach(), w.scale,
                                      causal, return_lse=True)
        dO = Gd.to(O.dtype)
        g_lib = spa.spa_attn_bwd(Q.detach(), K.detach(), V.detach(), P.detach(), O_lib, dO, lse,
                                 w.scale, causal, grad_dtype=Q.dtype)
    torch.cuda.synchronize()
    assert O.dtype == Q.dtype and torch.equal(O.detach(), O_lib)
    grads = [t.grad for t in leaves]
    for t, g in zip(leaves, grads):
        assert g is not None and g.shape == t.shape and g.dtype == t.dtype
    assert torch.equal(grads[1], g_lib[1]) and torch.equal(grads[2], g_lib[2])
    if dt == "f32":  # the fp32 backward has no atomics: every gradient bit for bit
        assert torch.equal(grads[0], g_lib[0]) and torch.equal(grads[3], g_lib[3])
    else:
        close("dQ vs library", f64(grads[0]), f64(g_lib[0]), 1e-2)
        close("dP vs library", f64(grads[3]), f64(g_lib[3].to(P.dtype)), 1e-2)
    tol = 2e-2 if dt == "bf16" else 1e-4

    ref = oracle.attn_bwd(x.Q, x.K, x.V, x.P, f64(dO.cpu()), w.scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV", "dP"), grads, ref):
        close(f"{name} vs oracle", f64(g), r, tol)


def test_autograd_plain_sum_and_projection_only(dev, oracle_mod):
    """O.sum().backward() (autograd hands over an expanded, non-contiguous ones tensor) with
    only P requiring a gradient: the projection's gradient alone, as when training P."""
    w = inputs.Workload("autograd-sum", 1, 2, 190, 128, 32, 128, True, seed=3301)
    x = inputs.draw(w)
    Q, K, V = (t.to(dev) for t in (x.Q, x.K, x.V))
    P = x.P.to(dev).requires_grad_(True)
    spa.spa_attention(Q, K, V, P, w.scale, True).sum().backward()
    torch.cuda.synchronize()
    ones = np.ones((w.B, w.H, w.N, w.dv))
    ref = oracle.attn_bwd(x.Q, x.K, x.V, x.P, ones, w.scale, True)
    close("dP vs oracle", f64(P.grad), ref[3], 2e-2)
