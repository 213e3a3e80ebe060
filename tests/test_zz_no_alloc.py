"""The allocation-free forward (spa_attn_fwd_noalloc, the library's static per-GPU workspace)
against the workspace-taking spa_attn_fwd on the same inputs, through the C ABI (MI355X
only): two calls in a row, the second smaller, each bit-equal to the reference call (same
kernels, same operands; only the workspace's address differs)."""
import sys

import pytest
import torch

import jl_feature_projected_amd as spa
from jl_feature_projected_amd import inputs

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a ROCm GPU"
    spa.lib()
    return torch.device("cuda:0")


def _pair(w, dev, out_dtype):
    x = inputs.draw(w)
    Q, K, V, P = (t.to(dev) for t in (x.Q, x.K, x.V, x.P))
    ws = torch.empty(spa.spa_attn_fwd_workspace_bytes(w.B, w.H, w.N, w.d, w.m, w.dv, Q.dtype),
                     dtype=torch.uint8, device=dev)
    ref, ref_lse = spa.spa_attn_fwd(Q, K, V, P, w.scale, w.causal, out_dtype=out_dtype,
                                    return_lse=True, workspace=ws)
    out = torch.empty_like(ref)
    lse = torch.empty_like(ref_lse)
    got = spa.spa_attn_fwd_noalloc(Q, K, V, P, w.scale, w.causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return ref, ref_lse, got, lse


CALLS = [  # first the benchmark's workload, then a smaller ragged one, then the fp32 path
    (inputs.WORKLOADS["c3"], torch.bfloat16),
    (inputs.Workload("noalloc-small", 1, 3, 1000, 64, 16, 64, False, seed=8100), torch.float32),
    (inputs.Workload("noalloc-f32", 1, 2, 333, 64, 16, 64, True, dtype="f32", seed=8101),
     torch.float32),
]


def test_noalloc_matches_workspace_forward(dev):
    assert spa.spa_attn_fwd_noalloc_max_workspace_bytes() == 128 << 20
    for w, odt in CALLS:
        note(f"{w.name} out={odt}")
        ref, ref_lse, got, lse = _pair(w, dev, odt)
        assert torch.equal(got.view(torch.int16) if odt == torch.bfloat16 else got.view(torch.int32),
                           ref.view(torch.int16) if odt == torch.bfloat16 else ref.view(torch.int32))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


def test_noalloc_rejects_sizes_beyond_its_scratch(dev):
    w = inputs.Workload("noalloc-big", 2, 16, 16384, 128, 32, 128, True, seed=8102)
    need = spa.spa_attn_fwd_workspace_bytes(w.B, w.H, w.N, w.d, w.m, w.dv, torch.bfloat16)
    assert need > spa.spa_attn_fwd_noalloc_max_workspace_bytes()
    Q = torch.zeros((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    V = torch.zeros((w.B, w.H, w.N, w.dv), dtype=torch.bfloat16, device=dev)
    P = torch.zeros((w.H, w.d, w.m), dtype=torch.bfloat16, device=dev)
    with pytest.raises(spa.SpaError) as e:
        spa.spa_attn_fwd_noalloc(Q, Q, V, P, w.scale, True)
    assert e.value.status == spa.SPA_ERR_UNSUPPORTED
