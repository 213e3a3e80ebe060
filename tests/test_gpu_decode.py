"""GPU parity of the decode path (spa_kcache_append, spa_attn_decode) through the C ABI.

Inputs are seeded workloads' stored bf16 bits: a length-Nk sequence's keys go into the
projected-key cache (fp16) with spa_kcache_append, its values into the value cache, and the
last Nq queries attend to the first Nk cache rows; the oracle evaluates the same rows of the
square forward in double from the same bits (queries at positions Nk - Nq .. Nk - 1).
Tolerance: max-abs 2e-2 on fp32 outputs (plus half a bf16 ulp on bf16 outputs), as for the
bf16 forward: the cache's fp16 rounding is the forward's, the rest is fp32.
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
    print(f"[gpu-decode] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a ROCm GPU"
    spa.lib()
    return torch.device("cuda:0")


def build_caches(x, w, rows, dev):
    K, V, P = (t.to(dev) for t in (x.K, x.V, x.P))
    cache = torch.zeros((w.B, w.H, rows, w.m), dtype=torch.float16, device=dev)
    spa.spa_kcache_append(K, P, cache, 0)
    Vc = torch.zeros((w.B, w.H, rows, w.dv), dtype=torch.bfloat16, device=dev)
    Vc[:, :, : w.N] = V
    return cache, Vc, P


def check(name, got, ref, out_bf16=False):
    err = np.abs(got - ref)
    allow = TOL + (np.abs(ref) * 2.0 ** -9 if out_bf16 else 0.0)
    note(f"{name}: max-abs {err.max():.3e} of max {np.abs(ref).max():.3e}")
    assert np.all(np.isfinite(got)), name
    assert np.all(err <= allow), (name, float(err.max()))


CASES = [  # B, H, Nq, Nk, rows, d, m, dv, causal
    (1, 2, 1, 1, 8, 128, 32, 128, True),
    (1, 2, 1, 1000, 1024, 128, 32, 128, True),
    (2, 3, 3, 777, 800, 64, 16, 64, True),
    (1, 2, 16, 300, 300, 128, 32, 128, False),
    (1, 2, 17, 2049, 2100, 128, 8, 128, True),
    (1, 1, 40, 5000, 5000, 128, 5, 64, True),
    (1, 2, 4, 4096, 4096, 64, 64, 64, False),
    (1, 2, 2, 65536, 65536, 128, 32, 128, True),
    (1, 1, 1, 3000, 3000, 128, 128, 128, True),
    (1, 2, 8, 1500, 1600, 128, 32, 128, True),
    (2, 1, 5, 700, 700, 64, 16, 64, False),
    (1, 2, 24, 1000, 1100, 128, 64, 64, True),
    (2, 1, 33, 3000, 3000, 128, 128, 128, True),
    (1, 2, 16, 777, 800, 64, 48, 128, False),
    (1, 1, 20, 500, 500, 64, 24, 64, True),
    (1, 1, 7, 600, 640, 128, 5, 128, False),
    # m in 72..96 with more than four queries: the matrix-core kernel's three-k-step instance
    (1, 2, 16, 1000, 1000, 128, 80, 128, True),
    (1, 1, 9, 700, 720, 64, 72, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_matches_oracle(dev, oracle_mod, case):
    B, H, Nq, Nk, rows, d, m, dv, causal = case
    w = inputs.Workload(f"dec-{'-'.join(map(str, case))}", B, H, Nk, d, m, dv, causal,
                        seed=4000 + Nk + m)
    x = inputs.draw(w)
    note(w.name)
    cache, Vc, P = build_caches(x, w, rows, dev)
    Q = x.Q[:, :, Nk - Nq:].contiguous().to(dev)
    O, lse = spa.spa_attn_decode(Q, cache, Vc, P, Nk, w.scale, causal, return_lse=True)
    torch.cuda.synchronize()
    Or, lr = oracle.attn_decode(x.Q[:, :, Nk - Nq:], x.K, x.V, x.P, w.scale, causal,
                                with_lse=True)
    check(w.name + " O", O.double().cpu().numpy(), Or)
    check(w.name + " lse", lse.double().cpu().numpy(), lr)


def test_decode_bf16_output_and_determinism(dev, oracle_mod):
    w = inputs.Workload("dec-bf16", 1, 4, 3000, 128, 32, 128, True, seed=4100)
    x = inputs.draw(w)
    cache, Vc, P = build_caches(x, w, 3000, dev)
    Q = x.Q[:, :, -3:].contiguous().to(dev)
    O1 = spa.spa_attn_decode(Q, cache, Vc, P, 3000, w.scale, True, out_dtype=torch.bfloat16)
    O2 = spa.spa_attn_decode(Q, cache, Vc, P, 3000, w.scale, True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
    Or = oracle.attn_decode(x.Q[:, :, -3:], x.K, x.V, x.P, w.scale, True)
    check("bf16 out", O1.double().cpu().numpy(), Or, out_bf16=True)


def test_kcache_append_values_and_untouched_rows(dev, oracle_mod):
    w = inputs.Workload("kcache", 2, 3, 333, 128, 40, 64, False, seed=4200)
    x = inputs.draw(w)
    K, P = x.K.to(dev), x.P.to(dev)
    rows, row0 = 400, 50
    cache = torch.full((2, 3, rows, 40), 7.0, dtype=torch.float16, device=dev)
    spa.spa_kcache_append(K, P, cache, row0)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    exact = oracle.project(x.K, x.P)
    mid = got[:, :, row0:row0 + 333].astype(np.float64)
    # fp32 accumulation of d products is within d * 2^-24 * sum |K_k P_kc| of the exact sum
    # (the standard recursive-summation bound), then one RNE step to fp16: half an fp16 ulp,
    # one whole ulp allowed for the case where the perturbed sum crossed a rounding boundary
    absum = oracle.project(np.abs(x.K.double().numpy()), np.abs(x.P.double().numpy()))
    ulp = np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64)
    allow = ulp + 128 * 2.0 ** -24 * absum
    diff = np.abs(mid - exact)
    rne = np.count_nonzero(mid != exact.astype(np.float16).astype(np.float64))
    note(f"append: {rne} of {diff.size} differ from RNE(exact); worst error / bound "
         f"{np.max(diff / allow):.3f}")
    assert np.all(diff <= allow)
    assert rne <= diff.size // 100
    assert np.all(got[:, :, :row0] == 7.0) and np.all(got[:, :, row0 + 333:] == 7.0)


def test_incremental_appends_match_one_shot(dev):
    w = inputs.Workload("kcache-inc", 1, 2, 1000, 64, 16, 64, True, seed=4300)
    x = inputs.draw(w)
    K, P, V = x.K.to(dev), x.P.to(dev), x.V.to(dev)
    one = torch.zeros((1, 2, 1024, 16), dtype=torch.float16, device=dev)
    spa.spa_kcache_append(K, P, one, 0)
    inc = torch.zeros_like(one)
    at = 0
    for n in (1, 7, 300, 1, 691):
        spa.spa_kcache_append(K[:, :, at:at + n].contiguous(), P, inc, at)
        at += n
    torch.cuda.synchronize()
    assert at == 1000 and torch.equal(one, inc)
    # a decode step after every append equals the prefix attention's last row
    Vc = torch.zeros((1, 2, 1024, 64), dtype=torch.bfloat16, device=dev)
    Vc[:, :, :1000] = V
    for nk in (1, 8, 308, 1000):
        Q = x.Q[:, :, nk - 1:nk].contiguous().to(dev)
        O = spa.spa_attn_decode(Q, inc, Vc, P, nk, w.scale, True)
        Or = oracle.attn_decode(x.Q[:, :, nk - 1:nk], x.K[:, :, :nk], x.V[:, :, :nk], x.P,
                                w.scale, True)
        check(f"step nk={nk}", O.double().cpu().numpy(), Or)


@pytest.mark.parametrize("key", ["c3", "c4"])
def test_decode_step_at_full_size(dev, oracle_mod, key):
    """One decode step (the last query of every head) against the whole cache of a full
    workload: every head checked against the oracle."""
    w = inputs.WORKLOADS[key]
    x = inputs.draw(w)
    note(f"{key} decode step, {w.B * w.H} heads x {w.N} keys")
    cache, Vc, P = build_caches(x, w, w.N, dev)
    Q = x.Q[:, :, -1:].contiguous().to(dev)
    O = spa.spa_attn_decode(Q, cache, Vc, P, w.N, w.scale, w.causal)
    torch.cuda.synchronize()
    Or = oracle.attn_decode(x.Q[:, :, -1:], x.K, x.V, x.P, w.scale, w.causal)
    check(f"{key} step", O.double().cpu().numpy(), Or)
