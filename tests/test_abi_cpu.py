"""The C ABI without a GPU: libspa.so loads, exports every symbol include/spa.h declares, and
rejects invalid calls on the host before any HIP call (so these run anywhere)."""
import ctypes
import os
import re

import pytest

import jl_feature_projected_amd as spa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spa.h")

# Fake, aligned, non-null device addresses far apart: every call below is rejected by host
# validation before a pointer could be used.
A, B_, C, D, E, F = (0x10000000 * k for k in range(1, 7))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return spa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(spa.EXPORTS)


def test_version_and_status_strings(L):
    assert L.spa_version() >= 100
    for code, name in ((0, "SPA_OK"), (1, "SPA_ERR_INVALID_ARGUMENT"), (2, "SPA_ERR_UNSUPPORTED"),
                       (3, "SPA_ERR_WORKSPACE"), (4, "SPA_ERR_HIP")):
        assert L.spa_status_string(code).decode() == name
    for code in (-1, 5, 99, 2 ** 31 - 1):
        assert L.spa_status_string(code).decode() == "SPA_ERR_UNKNOWN"


def _attn(L, **kw):
    a = dict(Q=A, K=B_, V=C, P=D, scale=0.125, causal=1, B=1, H=2, N=256, d=128, m=32, dv=128,
             dtype=spa.SPA_BF16, O=E, o_dtype=spa.SPA_F32, lse=None, ws=F, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return L.spa_attn_fwd(a["Q"], a["K"], a["V"], a["P"], a["scale"], a["causal"], a["B"],
                          a["H"], a["N"], a["d"], a["m"], a["dv"], a["dtype"], a["O"],
                          a["o_dtype"], a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(O=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(N=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(B=-1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(m=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(causal=2), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(o_dtype=9), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(Q=A + 2), spa.SPA_ERR_INVALID_ARGUMENT),           # misaligned
    (dict(lse=E + 2), spa.SPA_ERR_INVALID_ARGUMENT),         # misaligned lse
    (dict(O=A + 64), spa.SPA_ERR_INVALID_ARGUMENT),          # O overlaps Q
    (dict(lse=E + 16), spa.SPA_ERR_INVALID_ARGUMENT),        # lse overlaps O
    (dict(ws=E), spa.SPA_ERR_INVALID_ARGUMENT),              # workspace overlaps O
    (dict(ws_bytes=1024), spa.SPA_ERR_WORKSPACE),
    (dict(d=96), spa.SPA_ERR_UNSUPPORTED),
    (dict(dv=32), spa.SPA_ERR_UNSUPPORTED),
    (dict(m=129), spa.SPA_ERR_UNSUPPORTED),
    (dict(N=(1 << 22) + 1), spa.SPA_ERR_UNSUPPORTED),
    (dict(dtype=spa.SPA_F32, o_dtype=spa.SPA_BF16), spa.SPA_ERR_UNSUPPORTED),
    (dict(dtype=spa.SPA_F32, d=512), spa.SPA_ERR_UNSUPPORTED),
])
def test_attn_fwd_rejects_on_host(L, kw, code):
    assert _attn(L, **kw) == code
    assert len(L.spa_last_error()) > 0


def test_project_rejects_on_host(L):
    P = L.spa_project
    assert P(None, B_, C, 1, 1, 8, 64, 16, spa.SPA_BF16, None) == spa.SPA_ERR_INVALID_ARGUMENT
    assert P(A, B_, C, 1, 1, 0, 64, 16, spa.SPA_BF16, None) == spa.SPA_ERR_INVALID_ARGUMENT
    assert P(A, B_, C, 1, 1, 8, 80, 16, spa.SPA_BF16, None) == spa.SPA_ERR_UNSUPPORTED
    assert P(A, B_, C, 1, 1, 8, 64, 200, spa.SPA_BF16, None) == spa.SPA_ERR_UNSUPPORTED
    assert P(A, B_, A + 32, 1, 1, 8, 64, 16, spa.SPA_BF16, None) == spa.SPA_ERR_INVALID_ARGUMENT
    assert P(A + 4, B_, C, 1, 1, 8, 64, 16, spa.SPA_BF16, None) == spa.SPA_ERR_INVALID_ARGUMENT
    assert P(A, B_, C, 1, 1, 8, 64, 16, 5, None) == spa.SPA_ERR_INVALID_ARGUMENT


def test_workspace_bytes(L):
    # bf16: projected queries and keys at the padded width (m=8 -> 16 columns), one float
    # per (head, 256-key block) for the key norm maxima, then V^T in bf16 with rows padded
    # to a multiple of 64 keys
    n = L.spa_attn_fwd_workspace_bytes(2, 3, 100, 64, 8, 64, spa.SPA_BF16)
    one = 2 * 3 * 100 * 16 * 2
    a256 = lambda x: ((x + 255) // 256) * 256
    assert n == a256(a256(a256(one) + one) + 2 * 3 * 1 * 4) + 2 * 3 * 64 * 128 * 2
    n2 = L.spa_attn_fwd_workspace_bytes(1, 2, 1000, 128, 32, 128, spa.SPA_BF16)
    one2 = 2 * 1000 * 32 * 2
    assert n2 == a256(a256(a256(one2) + one2) + 2 * 4 * 4) + 2 * 128 * 1024 * 2
    n32 = L.spa_attn_fwd_workspace_bytes(1, 1, 512, 64, 16, 64, spa.SPA_F32)
    assert n32 == 2 * 512 * 16 * 4
    assert L.spa_attn_fwd_workspace_bytes(1, 1, 512, 96, 16, 64, spa.SPA_BF16) == 0
    assert L.spa_attn_fwd_workspace_bytes(0, 1, 512, 64, 16, 64, spa.SPA_BF16) == 0


def test_attn_fwd_plan(L):
    B = spa.SPA_BF16
    both = spa.SPA_PLAN_QUERIES_IN_ATTENTION | spa.SPA_PLAN_V_ROW_MAJOR
    # one-wave variant (m <= 32, >= 512 workgroups of 256 queries): projects the queries
    # itself; reads V as given when dv = 128
    assert L.spa_attn_fwd_plan(2, 16, 8192, 128, 32, 128, B, 1) == both
    assert L.spa_attn_fwd_plan(1, 128, 1024, 128, 32, 64, B, 0) == spa.SPA_PLAN_QUERIES_IN_ATTENTION
    assert L.spa_attn_fwd_plan(2, 64, 777, 64, 5, 128, B, 0) == both
    # two-wave variant: too few workgroups, or m > 32
    assert L.spa_attn_fwd_plan(4, 12, 2048, 64, 16, 64, B, 1) == 0
    assert L.spa_attn_fwd_plan(2, 16, 8192, 128, 64, 128, B, 1) == 0
    assert L.spa_attn_fwd_plan(2, 16, 8192, 128, 32, 128, spa.SPA_F32, 1) == 0
    # rejected arguments
    assert L.spa_attn_fwd_plan(2, 16, 8192, 96, 32, 128, B, 1) == -1
    assert L.spa_attn_fwd_plan(2, 16, 8192, 128, 32, 128, B, 2) == -1
    assert L.spa_attn_fwd_plan(0, 16, 8192, 128, 32, 128, B, 1) == -1


def test_profile_api_state(L):
    assert L.spa_profile_begin(0) == spa.SPA_ERR_INVALID_ARGUMENT
    d, e, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    assert L.spa_profile_end(ctypes.byref(d), ctypes.byref(e), ctypes.byref(n)) == \
        spa.SPA_ERR_INVALID_ARGUMENT


def test_binding_fails_loudly_without_device_tensors():
    import torch

    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    p = torch.zeros(1, 64, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        spa.spa_attn_fwd(x, x, x, p, 0.125, True)
    with pytest.raises(ValueError):
        spa.spa_project(x, p)


def _bwd(L, **kw):
    a = dict(Q=A, K=A + 0x100000, V=A + 0x200000, P=A + 0x300000, O=A + 0x400000,
             dO=A + 0x500000, lse=A + 0x600000, scale=0.125, causal=1, B=1, H=2, N=256,
             d=128, m=32, dv=128, dtype=spa.SPA_BF16, dQ=E, dK=E + 0x100000, dV=E + 0x200000,
             dP=E + 0x300000, g_dtype=spa.SPA_F32, ws=F, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.spa_attn_bwd(a["Q"], a["K"], a["V"], a["P"], a["O"], a["dO"], a["lse"], a["scale"],
                          a["causal"], a["B"], a["H"], a["N"], a["d"], a["m"], a["dv"],
                          a["dtype"], a["dQ"], a["dK"], a["dV"], a["dP"], a["g_dtype"], a["ws"],
                          a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dO=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(lse=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(N=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(causal=3), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(g_dtype=4), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(dQ=E + 8), spa.SPA_ERR_INVALID_ARGUMENT),              # misaligned
    (dict(dK=E + 0x10), spa.SPA_ERR_INVALID_ARGUMENT),           # overlaps dQ
    (dict(dV=A + 0x40), spa.SPA_ERR_INVALID_ARGUMENT),           # overlaps Q
    (dict(ws_bytes=100), spa.SPA_ERR_WORKSPACE),
    (dict(dtype=spa.SPA_F32, g_dtype=spa.SPA_BF16), spa.SPA_ERR_UNSUPPORTED),  # fp32: fp32 grads
    (dict(dtype=spa.SPA_F32, d=300), spa.SPA_ERR_UNSUPPORTED),
    (dict(dtype=spa.SPA_F32, dv=129), spa.SPA_ERR_UNSUPPORTED),
    (dict(dtype=spa.SPA_F32, m=129), spa.SPA_ERR_UNSUPPORTED),
    (dict(dtype=spa.SPA_F32, ws_bytes=100), spa.SPA_ERR_WORKSPACE),
    (dict(dtype=spa.SPA_F32, dV=A + 0x40), spa.SPA_ERR_INVALID_ARGUMENT),  # overlaps Q (fp32)
    (dict(m=129), spa.SPA_ERR_UNSUPPORTED),
    (dict(d=96), spa.SPA_ERR_UNSUPPORTED),
    (dict(dv=32), spa.SPA_ERR_UNSUPPORTED),
])
def test_attn_bwd_rejects_on_host(L, kw, code):
    assert _bwd(L, **kw) == code
    assert len(L.spa_last_error()) > 0


def test_bwd_workspace_bytes(L):
    a256 = lambda x: ((x + 255) // 256) * 256
    BH, N, d, m, dv = 2, 100, 64, 8, 64
    mp, np_ = 16, 128
    rows = BH * N
    sizes = [rows * mp * 2, rows * mp * 2, BH * mp * np_ * 2, BH * mp * np_ * 2, BH * dv * np_ * 2,
             BH * np_ * 2 * 4, rows * mp * 4, rows * mp * 4, BH * 1 * d * m * 4]
    assert L.spa_attn_bwd_workspace_bytes(1, 2, N, d, m, dv, spa.SPA_BF16) == sum(a256(s) for s in sizes)
    assert L.spa_attn_bwd_workspace_bytes(1, 2, N, d, 129, dv, spa.SPA_BF16) == 0
    # fp32 path: projected queries, keys and their gradients (fp32, m wide), then D
    f32 = [rows * m * 4] * 4 + [rows * 4]
    assert L.spa_attn_bwd_workspace_bytes(1, 2, N, d, m, dv, spa.SPA_F32) == sum(a256(s) for s in f32)
    assert L.spa_attn_bwd_workspace_bytes(1, 2, N, 96, 5, 40, spa.SPA_F32) == \
        sum(a256(s) for s in [rows * 5 * 4] * 4 + [rows * 4])
    assert L.spa_attn_bwd_workspace_bytes(1, 2, N, 300, m, dv, spa.SPA_F32) == 0
    assert L.spa_attn_bwd_workspace_bytes(1, 2, N, d, 129, dv, spa.SPA_F32) == 0


def _decode(L, **kw):
    a = dict(Q=A, cache=B_, Vc=C, P=D, scale=0.125, causal=1, B=1, H=2, Nq=1, Nk=4096,
             rows=8192, d=128, m=32, dv=128, dtype=spa.SPA_BF16, O=E, o_dtype=spa.SPA_F32,
             lse=None, ws=F, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.spa_attn_decode(a["Q"], a["cache"], a["Vc"], a["P"], a["scale"], a["causal"],
                             a["B"], a["H"], a["Nq"], a["Nk"], a["rows"], a["d"], a["m"],
                             a["dv"], a["dtype"], a["O"], a["o_dtype"], a["lse"], a["ws"],
                             a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(cache=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(Nq=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(Nq=5000), spa.SPA_ERR_INVALID_ARGUMENT),          # Nq > Nk
    (dict(Nk=9000), spa.SPA_ERR_INVALID_ARGUMENT),          # Nk > rows
    (dict(causal=2), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(dtype=spa.SPA_F32), spa.SPA_ERR_UNSUPPORTED),
    (dict(d=96), spa.SPA_ERR_UNSUPPORTED),
    (dict(m=129), spa.SPA_ERR_UNSUPPORTED),
    (dict(dv=96), spa.SPA_ERR_UNSUPPORTED),
    (dict(o_dtype=7), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(Q=A + 8), spa.SPA_ERR_INVALID_ARGUMENT),          # misaligned
    (dict(O=B_), spa.SPA_ERR_INVALID_ARGUMENT),             # O overlaps the cache
    (dict(ws_bytes=16), spa.SPA_ERR_WORKSPACE),
    (dict(ws=E), spa.SPA_ERR_INVALID_ARGUMENT),             # workspace overlaps O
])
def test_attn_decode_rejects_on_host(L, kw, code):
    assert _decode(L, **kw) == code
    assert len(L.spa_last_error()) > 0


def test_kcache_append_rejects_on_host(L):
    ok = dict(K=A, P=B_, cache=C, B=1, H=2, N=16, d=128, m=32, rows=64, row0=0,
              dtype=spa.SPA_BF16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.spa_kcache_append(a["K"], a["P"], a["cache"], a["B"], a["H"], a["N"], a["d"],
                                   a["m"], a["rows"], a["row0"], a["dtype"], None)
    for kw, code in ((dict(K=None), spa.SPA_ERR_INVALID_ARGUMENT),
                     (dict(row0=49), spa.SPA_ERR_INVALID_ARGUMENT),   # past the cache end
                     (dict(row0=-1), spa.SPA_ERR_INVALID_ARGUMENT),
                     (dict(dtype=spa.SPA_F32), spa.SPA_ERR_UNSUPPORTED),
                     (dict(d=32), spa.SPA_ERR_UNSUPPORTED),
                     (dict(m=200), spa.SPA_ERR_UNSUPPORTED),
                     (dict(cache=A), spa.SPA_ERR_INVALID_ARGUMENT),   # overlaps K
                     (dict(P=B_ + 4), spa.SPA_ERR_INVALID_ARGUMENT)):
        assert call(**kw) == code, kw


def test_decode_workspace_bytes(L):
    # B*H*Nq*nsplit*(dv+2) floats; nsplit from the split rule (about 1024 workgroups, at
    # least two 256-key blocks per split when the cache has two): 32 heads, one query,
    # 32768 keys -> 32 splits of 1024 keys; 8192 keys -> 16 splits of 512 (not 32 of 256)
    assert L.spa_attn_decode_workspace_bytes(1, 32, 1, 32768, 128) == 32 * 1 * 32 * 130 * 4
    assert L.spa_attn_decode_workspace_bytes(2, 16, 1, 8192, 128) == 32 * 1 * 16 * 130 * 4
    assert L.spa_attn_decode_workspace_bytes(1, 1, 1, 100, 64) == 1 * 1 * 1 * 66 * 4
    assert L.spa_attn_decode_workspace_bytes(1, 2, 17, 16, 128) == 0  # Nq > Nk


def test_sfa_fwd_rejects_on_host(L):
    ok = dict(Q=A, K=B_, V=C, topk=16, scale=0.125, causal=1, B=1, H=2, N=256, d=128, dv=128,
              dtype=spa.SPA_BF16, O=E, o_dtype=spa.SPA_F32, lse=None, ws=F, ws_bytes=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.spa_sfa_fwd(a["Q"], a["K"], a["V"], a["topk"], a["scale"], a["causal"], a["B"],
                             a["H"], a["N"], a["d"], a["dv"], a["dtype"], a["O"], a["o_dtype"],
                             a["lse"], a["ws"], a["ws_bytes"], None)
    for kw, code in ((dict(Q=None), spa.SPA_ERR_INVALID_ARGUMENT),
                     (dict(topk=0), spa.SPA_ERR_INVALID_ARGUMENT),
                     (dict(topk=129), spa.SPA_ERR_INVALID_ARGUMENT),
                     (dict(causal=3), spa.SPA_ERR_INVALID_ARGUMENT),
                     (dict(dtype=spa.SPA_F32), spa.SPA_ERR_UNSUPPORTED),
                     (dict(d=96, topk=8), spa.SPA_ERR_UNSUPPORTED),
                     (dict(dv=32), spa.SPA_ERR_UNSUPPORTED),
                     (dict(O=A), spa.SPA_ERR_INVALID_ARGUMENT),
                     (dict(ws_bytes=100), spa.SPA_ERR_WORKSPACE),
                     (dict(V=C + 2), spa.SPA_ERR_INVALID_ARGUMENT)):
        assert call(**kw) == code, kw
        assert len(L.spa_last_error()) > 0
    # the forward's workspace with m = d
    assert L.spa_sfa_fwd_workspace_bytes(1, 2, 256, 128, 128) == \
        L.spa_attn_fwd_workspace_bytes(1, 2, 256, 128, 128, 128, spa.SPA_BF16)
    assert L.spa_sfa_fwd_workspace_bytes(1, 2, 256, 96, 128) == 0


def test_binding_rejects_tensors_on_other_devices():
    """The kernels run on the first tensor's device; the binding refuses any other."""
    from types import SimpleNamespace as T
    spa._same_device(T(device="cuda:0"), T(device="cuda:0"), None)
    with pytest.raises(ValueError):
        spa._same_device(T(device="cuda:0"), T(device="cuda:0"), T(device="cuda:1"))


def test_probe_rates_rejects_null_outputs(L):
    x = ctypes.c_double()
    st = L.spa_probe_rates(None, ctypes.byref(x), ctypes.byref(x), ctypes.byref(x), None)
    assert st == spa.SPA_ERR_INVALID_ARGUMENT
    assert b"null" in L.spa_last_error()
