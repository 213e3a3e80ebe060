"""GPU parity of the backward (spa_attn_bwd) against the oracle's backward (MI355X only).

Inputs are the seeded workloads' stored bf16 bits, dO a seeded N(0, 1) draw; the forward
runs on the GPU (its bf16 output and lse feed the backward, as in training), the oracle
computes the exact gradients in double from the same stored bits.

Tolerance, per gradient tensor g: max |g_gpu - g_ref| <= 2e-2 * max |g_ref|. Budget: the
weights are recomputed from fp16 projected operands (the forward's), meet dO in bf16
(2^-9 relative) and dS meets the projected operands in fp16 (2^-11); D uses the forward's
bf16 output (2^-9 relative per term); all sums are fp32 MFMA accumulations. Measured on
MI355X: 1.4e-3 to 8.2e-3 of the largest entry (the worst at m = 5, where the fewest
projected features carry the most rounding per score); 2e-2 leaves a margin of 2.4x.
"""
import math
import sys

import numpy as np
import pytest
import torch

import jl_feature_projected_amd as spa
import oracle
from jl_feature_projected_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def note(msg):
    print(f"[gpu-bwd] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a ROCm GPU"
    spa.lib()
    return torch.device("cuda:0")


def run_bwd(w, dev, seed, g_dtype=torch.float32, ones_v=False, zero_do=False):
    x = inputs.draw(w)
    dO = inputs.draw_grad_output(w, seed)
    V = torch.ones_like(x.V) if ones_v else x.V
    if zero_do:
        dO = torch.zeros_like(dO)
    Q, K, Vd, P, dOd = (t.to(dev) for t in (x.Q, x.K, V, x.P, dO))
    O, lse = spa.spa_attn_fwd(Q, K, Vd, P, w.scale, w.causal, out_dtype=torch.bfloat16,
                              return_lse=True)
    g = spa.spa_attn_bwd(Q, K, Vd, P, O, dOd, lse, w.scale, w.causal, grad_dtype=g_dtype)
    torch.cuda.synchronize()
    return x, V, dO, [t.float().cpu().numpy().astype(np.float64) for t in g]


def compare(name, got, ref):
    err = np.max(np.abs(got - ref))
    top = np.max(np.abs(ref))
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    note(f"{name}: max-abs {err:.3e} of max {top:.3e} ({err / top:.2e} relative), frobenius {fro:.2e}")
    assert np.all(np.isfinite(got)), name
    assert err <= TOL * top, name


SMALL = [  # B, H, N, d, m, dv, causal
    (1, 2, 100, 64, 16, 64, True),
    (2, 2, 257, 128, 32, 128, True),
    (1, 2, 300, 128, 32, 128, False),
    (1, 1, 513, 64, 64, 64, True),
    (1, 3, 64, 128, 8, 128, False),
    (2, 1, 1000, 128, 32, 128, True),
    (1, 2, 777, 128, 5, 64, True),
    (1, 2, 300, 128, 128, 128, True),
    (2, 1, 333, 64, 100, 64, False),
    (1, 1, 200, 128, 128, 64, False),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "-".join(map(str, s)))
def test_backward_small_shapes(dev, oracle_mod, shape):
    B, H, N, d, m, dv, causal = shape
    w = inputs.Workload(f"bwd-{N}", B, H, N, d, m, dv, causal, seed=900 + N)
    x, V, dO, got = run_bwd(w, dev, seed=31 + N)
    ref = oracle.attn_bwd(x.Q, x.K, V, x.P, dO, w.scale, causal)
    for name, a, b in zip(("dQ", "dK", "dV", "dP"), got, ref):
        compare(f"{shape} {name}", a, b)


# Wider grids (128 heads, 512 or more blocks of 256 keys, as the longer workloads launch) at
# ragged N, both masks, m not a multiple of 16, d = 64 and 128, dv = 64 and 128, every head
# against the oracle.
WIDE = [  # B, H, N, d, m, dv, causal
    (4, 32, 1000, 64, 24, 64, True),
    (2, 64, 777, 128, 5, 128, False),
    (1, 128, 1025, 128, 32, 128, True),
    (4, 32, 1024, 128, 16, 64, False),
]


@pytest.mark.parametrize("shape", WIDE, ids=lambda s: "-".join(map(str, s)))
def test_backward_wide_grids(dev, oracle_mod, shape):
    B, H, N, d, m, dv, causal = shape
    w = inputs.Workload(f"bwd-wide-{N}", B, H, N, d, m, dv, causal, seed=1900 + N + m)
    x, V, dO, got = run_bwd(w, dev, seed=41 + N)
    ref = oracle.attn_bwd(x.Q, x.K, V, x.P, dO, w.scale, causal)
    for name, a, b in zip(("dQ", "dK", "dV", "dP"), got, ref):
        compare(f"{shape} {name}", a, b)


def test_backward_headline_recipe_reduced_length(dev, oracle_mod):
    """The N = 8192 workload's recipe (low-rank-plus-noise Q and K, d = dv = 128, m = 32,
    causal) on two heads at N = 2048, where the double-precision oracle takes seconds."""
    w = inputs.WORKLOADS["c3"].replace(B=1, H=2, N=2048)
    x, V, dO, got = run_bwd(w, dev, seed=77)
    ref = oracle.attn_bwd(x.Q, x.K, V, x.P, dO, w.scale, True)
    for name, a, b in zip(("dQ", "dK", "dV", "dP"), got, ref):
        compare(f"c3-recipe N=2048 {name}", a, b)


def test_backward_identity_projection_d128(dev, oracle_mod):
    """m = d = 128 with P = I: the gradients of exact attention (the P = I workload's shape)."""
    w = inputs.Workload("bwd-identity-128", 1, 2, 300, 128, 128, 128, True, proj="identity",
                        seed=6)
    x, V, dO, got = run_bwd(w, dev, seed=7)
    ref = oracle.attn_bwd(x.Q, x.K, V, x.P, dO, w.scale, True)
    for name, g, r in zip(("dQ", "dK", "dV", "dP"), got, ref):
        compare("identity-128 " + name, g, r)


def test_backward_identity_projection(dev, oracle_mod):
    w = inputs.Workload("bwd-identity", 1, 2, 400, 64, 64, 64, True, proj="identity", seed=4)
    x, V, dO, got = run_bwd(w, dev, seed=5)
    ref = oracle.attn_bwd(x.Q, x.K, V, x.P, dO, w.scale, True)
    for name, a, b in zip(("dQ", "dK", "dV", "dP"), got, ref):
        compare(f"identity {name}", a, b)


def test_backward_closed_forms(dev):
    w = inputs.Workload("bwd-closed", 1, 2, 300, 128, 32, 128, True, seed=8)
    # dO = 0: every gradient is exactly zero
    _, _, _, g = run_bwd(w, dev, seed=1, zero_do=True)
    assert all(np.all(t == 0.0) for t in g)
    # V = 1: O does not depend on the scores, so dQ, dK, dP vanish (up to the rounding of
    # D = <dO, O> against <dO, V_j>, both exact here since O = 1 is representable)
    _, _, _, g = run_bwd(w, dev, seed=2, ones_v=True)
    for name, t in zip(("dQ", "dK", "dP"), (g[0], g[1], g[3])):
        assert np.max(np.abs(t)) <= 1e-3, name


def test_backward_bf16_gradients_and_determinism(dev):
    # dK and dV are bit-identical run to run; dQ and dP come from the projected-query
    # gradient, which the key-major kernel accumulates by fp32 atomic adds in an order that
    # varies between runs, so they agree to rounding: the fp32 sums to a few ulps, which a
    # bf16 rounding of dQ can turn into one bf16 ulp of the element.
    w = inputs.Workload("bwd-bf16", 1, 2, 600, 128, 32, 128, True, seed=9)
    _, _, _, g32 = run_bwd(w, dev, seed=3)
    _, _, _, g16 = run_bwd(w, dev, seed=3, g_dtype=torch.bfloat16)
    _, _, _, g16b = run_bwd(w, dev, seed=3, g_dtype=torch.bfloat16)
    for name, a, b, c in zip(("dQ", "dK", "dV", "dP"), g16, g32, g16b):
        if name in ("dK", "dV"):
            assert np.array_equal(a, c), name  # bit-identical reruns
        elif name == "dQ":
            assert np.all(np.abs(a - c) <= 2 ** -8 * np.abs(c) + 1e-30), name
        else:
            assert np.max(np.abs(a - c)) <= 1e-5 * np.max(np.abs(c)), name
        assert np.max(np.abs(a - b)) <= 2 ** -8 * np.max(np.abs(b)) + 1e-30, name


def test_backward_full_headline_size_two_heads_exact(dev, oracle_mod):
    """The whole N = 8192 workload (all 32 heads, the launch the benchmark times, dO as the
    benchmark draws it); the oracle's exact backward for head 0 of both batches (the two
    (b, h) pairs that share P[0], so dP[0] is comparable too), every element compared."""
    w = inputs.WORKLOADS["c3"]
    x, V, dO, g = run_bwd(w, dev, seed=w.seed + 1)
    assert all(np.all(np.isfinite(t)) for t in g)
    sel = [0, w.H]  # (b, h) = (0, 0) and (1, 0) in the flattened [B*H] order
    flat = lambda t, last: t.reshape(w.B * w.H, w.N, last)[sel].reshape(2, 1, w.N, last)
    Q2, K2 = flat(x.Q, w.d), flat(x.K, w.d)
    V2, dO2 = flat(V, w.dv), flat(dO, w.dv)
    P0 = x.P[:1]
    ref = oracle.attn_bwd(Q2, K2, V2, P0, dO2, w.scale, True)
    got = [flat(torch.from_numpy(g[0]), w.d).numpy(), flat(torch.from_numpy(g[1]), w.d).numpy(),
           flat(torch.from_numpy(g[2]), w.dv).numpy(), g[3][:1]]
    for name, a, b in zip(("dQ", "dK", "dV", "dP"), got, ref):
        compare(f"c3 full size, head 0 of both batches: {name}", a, b)
