"""GPU parity of the fp32 backward (spa_attn_bwd with fp32 inputs) against the oracle's
backward (MI355X only).

The fp32 forward runs on the GPU first (its fp32 output and lse feed the backward, as in
training); the oracle computes the exact gradients in double from the same stored fp32
inputs and dO.

Tolerance, per gradient tensor g: max |g_gpu - g_ref| <= 1e-4 * max |g_ref| (the fp32
path's bound). Budget: every product and sum is fp32 (2^-24 relative per operation), the
projections and the forward's O and lse carry one such rounding each, and the longest sums
run over N keys or B*N tokens; the measured errors are near 1e-6.
"""
import sys

import numpy as np
import pytest
import torch

import jl_feature_projected_amd as spa
from jl_feature_projected_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-4


def note(msg):
    print(f"[gpu-bwd-f32] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a ROCm GPU"
    spa.lib()
    return torch.device("cuda:0")


def run(w, dev, seed):
    x = inputs.draw(w)
    dO = inputs.draw_grad_output(w, seed)
    assert x.Q.dtype == torch.float32 and dO.dtype == torch.float32
    Q, K, V, P, dOd = (t.to(dev) for t in (x.Q, x.K, x.V, x.P, dO))
    O, lse = spa.spa_attn_fwd(Q, K, V, P, w.scale, w.causal, return_lse=True)
    assert O.dtype == torch.float32
    g = spa.spa_attn_bwd(Q, K, V, P, O, dOd, lse, w.scale, w.causal)
    torch.cuda.synchronize()
    return x, dO, [t.cpu().numpy().astype(np.float64) for t in g]


def compare(name, got, ref):
    err = np.max(np.abs(got - ref))
    top = np.max(np.abs(ref))
    note(f"{name}: max-abs {err:.3e} of max {top:.3e} ({err / max(top, 1e-300):.2e} relative)")
    assert np.all(np.isfinite(got)), name
    assert err <= TOL * top or err == 0.0, name


def check(w, dev, oracle_mod, seed):
    x, dO, g = run(w, dev, seed)
    ref = oracle_mod.attn_bwd(x.Q, x.K, x.V, x.P, dO, w.scale, w.causal)
    for name, a, b in zip(("dQ", "dK", "dV", "dP"), g, ref):
        compare(f"{w.name}: {name}", a, b)
    return g, ref


def test_backward_f32_workload(dev, oracle_mod):
    """The fp32 workload (one head, N = 512, d = 64, m = 16, dv = 64, non-causal), in full."""
    w = inputs.WORKLOADS["c1"]
    check(w, dev, oracle_mod, seed=w.seed + 1)


SHAPES = [  # B, H, N, d, m, dv, causal
    (2, 3, 100, 96, 5, 40, True),
    (1, 2, 257, 128, 128, 128, True),
    (1, 2, 300, 256, 64, 128, False),
    (2, 1, 33, 64, 33, 64, True),
    (1, 2, 700, 64, 16, 64, True),
    (1, 1, 64, 48, 1, 1, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_backward_f32_shapes(dev, oracle_mod, shape):
    B, H, N, d, m, dv, causal = shape
    w = inputs.Workload(f"bwd-f32-{'-'.join(map(str, shape))}", B, H, N, d, m, dv, causal,
                        dtype="f32", seed=4000 + N + m)
    check(w, dev, oracle_mod, seed=17)


def test_backward_f32_single_token(dev, oracle_mod):
    """N = 1, causal: the one weight is 1, so dS = 0 (dQ = dK = dP = 0) and dV = dO (up to
    the fp32 rounding of the recomputed weight)."""
    w = inputs.Workload("bwd-f32-n1", 1, 2, 1, 64, 16, 64, True, dtype="f32", seed=5)
    x, dO, g = run(w, dev, seed=6)
    top = np.max(np.abs(dO.numpy()))
    for name, t in zip(("dQ", "dK", "dP"), (g[0], g[1], g[3])):
        assert np.max(np.abs(t)) <= 1e-6 * max(1.0, top), name
    assert np.max(np.abs(g[2] - dO.numpy())) <= 1e-6 * top


def test_backward_f32_deterministic(dev):
    w = inputs.Workload("bwd-f32-det", 2, 2, 300, 64, 16, 64, True, dtype="f32", seed=8)
    _, _, a = run(w, dev, seed=9)
    _, _, b = run(w, dev, seed=9)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
