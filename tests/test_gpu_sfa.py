"""GPU parity of sparse feature attention (spa_sfa_fwd) against the oracle (MI355X only).

The oracle selects each row's Top-k features in float64 (ties: lower index first) and runs
the exact forward with P = I; the GPU selects on the stored bf16 bits and runs the streamed
attention kernel on fp16 operands. A different selection anywhere would move an output by
far more than the tolerance, so agreement also checks the selection. Tolerance: max-abs
2e-2 on fp32 outputs, as for the bf16 forward.
"""
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
    print(f"[gpu-sfa] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a ROCm GPU"
    spa.lib()
    return torch.device("cuda:0")


def check(name, got, ref):
    err = np.abs(got - ref)
    note(f"{name}: max-abs {err.max():.3e} of max {np.abs(ref).max():.3e}")
    assert np.all(np.isfinite(got)), name
    assert err.max() <= TOL, (name, float(err.max()))


CASES = [  # B, H, N, d, dv, topk, causal
    (1, 2, 300, 128, 128, 16, True),
    (2, 1, 777, 64, 64, 8, False),
    (1, 2, 1000, 128, 64, 1, True),
    (1, 1, 513, 128, 128, 128, True),
    (1, 2, 200, 64, 128, 64, False),
    (1, 3, 129, 128, 128, 5, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_sfa_matches_oracle(dev, oracle_mod, case):
    B, H, N, d, dv, k, causal = case
    w = inputs.Workload(f"sfa-{'-'.join(map(str, case))}", B, H, N, d, d, dv, causal,
                        proj="identity", seed=5000 + N + k)
    x = inputs.draw(w)
    note(w.name)
    Q, K, V = (t.to(dev) for t in (x.Q, x.K, x.V))
    O, lse = spa.spa_sfa_fwd(Q, K, V, k, w.scale, causal, return_lse=True)
    torch.cuda.synchronize()
    Or, lr = oracle.sfa_fwd(x.Q, x.K, x.V, k, w.scale, causal, with_lse=True)
    check(w.name + " O", O.double().cpu().numpy(), Or)
    check(w.name + " lse", lse.double().cpu().numpy(), lr)


def test_sfa_ties_follow_the_index_order(dev, oracle_mod):
    """Rows built from few distinct magnitudes: the selection is decided by the tie reading."""
    B, H, N, d, dv, k = 1, 2, 256, 128, 64, 12
    rng = np.random.default_rng(77)
    vals = np.array([0.5, 1.0, 1.5, 2.0])
    Qn = rng.choice(vals, size=(B, H, N, d)) * rng.choice([-1.0, 1.0], size=(B, H, N, d))
    Kn = rng.choice(vals, size=(B, H, N, d)) * rng.choice([-1.0, 1.0], size=(B, H, N, d))
    Vn = rng.standard_normal((B, H, N, dv))
    Q, K, V = (inputs.to_storage(a, "bf16") for a in (Qn, Kn, Vn))
    O = spa.spa_sfa_fwd(Q.to(dev), K.to(dev), V.to(dev), k, 0.125, True)
    torch.cuda.synchronize()
    Or = oracle.sfa_fwd(Q, K, V, k, 0.125, True)
    check("ties", O.double().cpu().numpy(), Or)


def test_sfa_headline_shape_sampled(dev, oracle_mod):
    """The N = 8192 workload's inputs at d = 128 with k = 16, every head, sampled rows."""
    w = inputs.WORKLOADS["c3"]
    x = inputs.draw(w)
    k = 16
    Q, K, V = (t.to(dev) for t in (x.Q, x.K, x.V))
    O = spa.spa_sfa_fwd(Q, K, V, k, w.scale, True)
    torch.cuda.synchronize()
    Qs, Ks = oracle.topk_features(x.Q, k), oracle.topk_features(x.K, k)
    BH = w.B * w.H
    rng = np.random.default_rng(3)
    rows = np.concatenate([[0, 1, 63, 64, 127, 128, 8191], rng.integers(0, w.N, 9)])
    rb = np.repeat(np.arange(BH), len(rows))
    ri = np.tile(rows, BH)
    eye = np.broadcast_to(np.eye(w.d), (w.H, w.d, w.d)).copy()
    Or = oracle.attn_rows(Qs, Ks, x.V, eye, w.scale, True, rb, ri)
    got = O.reshape(BH, w.N, w.dv)[torch.from_numpy(rb), torch.from_numpy(ri)]
    check("c3 k=16 sampled", got.double().cpu().numpy(), Or)


def _selected_rows(ws, BH, N, d):
    """The fp16 query and key rows spa_sfa_fwd leaves in its workspace: [BH, N, d] each, the
    queries first, the keys at the next 256-byte boundary."""
    n = BH * N * d * 2
    k_off = (n + 255) // 256 * 256
    q = ws[:n].view(torch.float16).reshape(BH, N, d)
    k = ws[k_off:k_off + n].view(torch.float16).reshape(BH, N, d)
    return q.cpu(), k.cpu()


SELECT = [  # workload or shape, topk
    ("c3", 16), ("c3", 1), ((1, 3, 257, 64), 5), ((2, 2, 300, 128), 64), ((1, 1, 100, 128), 128),
]


@pytest.mark.parametrize("case", SELECT, ids=lambda c: f"{c[0] if isinstance(c[0], str) else '-'.join(map(str, c[0]))}-k{c[1]}")
def test_sfa_selection_bit_exact(dev, oracle_mod, case):
    """The Top-k support the GPU selects (the nonzero features of the fp16 rows in the
    workspace) equals the oracle's selection bit for bit, ties included (lower index first),
    and each kept value is the round-to-nearest-even fp16 of the input times the query
    scale (scale * log2 e) or 1 for keys. Scaling Attention via Feature Sparsity notes, key
    design 1 (the Topk operator)."""
    src, k = case
    if isinstance(src, str):
        w = inputs.WORKLOADS[src]
        x = inputs.draw(w)
        B, H, N, d, dv = w.B, w.H, w.N, w.d, w.dv
        Qc, Kc, Vc, scale = x.Q, x.K, x.V, w.scale
    else:
        B, H, N, d = src
        dv = 64
        w = inputs.Workload("sel", B, H, N, d, d, dv, True, proj="identity", seed=6000 + N + k)
        x = inputs.draw(w)
        Qc, Kc, Vc, scale = x.Q, x.K, x.V, w.scale
    note(f"selection {case}")
    ws = torch.empty(spa.spa_sfa_fwd_workspace_bytes(B, H, N, d, dv), dtype=torch.uint8,
                     device=dev)
    spa.spa_sfa_fwd(Qc.to(dev), Kc.to(dev), Vc.to(dev), k, scale, True, workspace=ws)
    torch.cuda.synchronize()
    gq, gk = _selected_rows(ws, B * H, N, d)
    qscale = np.float32(scale) * np.float32(1.44269504088896340736)
    for name, X, got, mult in (("Q", Qc, gq, qscale), ("K", Kc, gk, np.float32(1.0))):
        ref_sel = oracle.topk_features(X, k).reshape(B * H, N, d)
        X32 = X.float().reshape(B * H, N, d)
        want = torch.where(torch.from_numpy(ref_sel != 0), (X32 * float(mult)).half(),
                           torch.zeros((), dtype=torch.float16))
        # (a kept value whose fp16 rounding is zero counts as unkept on both sides)
        sup_ref = (want != 0).numpy()
        sup_got = (got != 0).numpy()
        bad = int(np.count_nonzero(sup_ref != sup_got))
        note(f"{name}: {B * H * N} rows, support mismatches {bad}")
        assert bad == 0, (name, bad)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), name


def test_sfa_selection_ties_bit_exact(dev, oracle_mod):
    """Rows of few distinct magnitudes: the tie rule decides most of the selection."""
    B, H, N, d, dv, k = 1, 2, 256, 128, 64, 12
    rng = np.random.default_rng(78)
    vals = np.array([0.5, 1.0, 1.5, 2.0])
    Qn = rng.choice(vals, size=(B, H, N, d)) * rng.choice([-1.0, 1.0], size=(B, H, N, d))
    Kn = rng.choice(vals, size=(B, H, N, d)) * rng.choice([-1.0, 1.0], size=(B, H, N, d))
    Vn = rng.standard_normal((B, H, N, dv))
    Q, K, V = (inputs.to_storage(a, "bf16") for a in (Qn, Kn, Vn))
    ws = torch.empty(spa.spa_sfa_fwd_workspace_bytes(B, H, N, d, dv), dtype=torch.uint8,
                     device=dev)
    spa.spa_sfa_fwd(Q.to(dev), K.to(dev), V.to(dev), k, 0.125, True, workspace=ws)
    torch.cuda.synchronize()
    gq, gk = _selected_rows(ws, B * H, N, d)
    for name, X, got in (("Q", Q, gq), ("K", K, gk)):
        sup_ref = oracle.topk_features(X, k).reshape(B * H, N, d) != 0
        assert np.array_equal(sup_ref, (got != 0).numpy()), name
