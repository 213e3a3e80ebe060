"""Feature-axis projected softmax attention (SPA / PDA style) on MI355X (gfx950).

A thin binding over the C ABI of ``libspa.so`` (declared in ``include/spa.h``). It only
marshals arguments: every step of the computation runs in the library's HIP kernels on the
caller's current torch stream. PyTorch provides device memory and streams. There is no
fallback: without the built library, or on tensors that are not on a ROCm device, calls raise.

    O = spa_attn_fwd(Q, K, V, P, scale, causal)      # Q,K [B,H,N,d], V [B,H,N,dv], P [H,d,m]
    Qt = spa_project(Q, P)                           # [B,H,N,m]
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspa.so")

SPA_OK = 0
SPA_ERR_INVALID_ARGUMENT = 1
SPA_ERR_UNSUPPORTED = 2
SPA_ERR_WORKSPACE = 3
SPA_ERR_HIP = 4
SPA_F32 = 0
SPA_BF16 = 1

EXPORTS = ("spa_version", "spa_status_string", "spa_last_error", "spa_project",
           "spa_attn_fwd_workspace_bytes", "spa_attn_fwd", "spa_attn_bwd_workspace_bytes",
           "spa_attn_bwd", "spa_sfa_fwd_workspace_bytes", "spa_sfa_fwd", "spa_kcache_append", "spa_attn_decode_workspace_bytes",
           "spa_attn_decode", "spa_profile_begin", "spa_profile_end", "spa_probe_rates",
           "spa_attn_fwd_noalloc", "spa_attn_fwd_noalloc_max_workspace_bytes",
           "spa_attn_fwd_plan")
SPA_PLAN_QUERIES_IN_ATTENTION = 1
SPA_PLAN_V_ROW_MAJOR = 2


class SpaError(RuntimeError):
    """A libspa call returned a status other than SPA_OK."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_STATUS_NAMES = {0: "SPA_OK", 1: "SPA_ERR_INVALID_ARGUMENT", 2: "SPA_ERR_UNSUPPORTED",
                 3: "SPA_ERR_WORKSPACE", 4: "SPA_ERR_HIP"}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libspa.so with its C signatures declared; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m jl_feature_projected_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, z, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_int
    L.spa_version.restype = i
    L.spa_version.argtypes = []
    L.spa_status_string.restype = ctypes.c_char_p
    L.spa_status_string.argtypes = [st]
    L.spa_last_error.restype = ctypes.c_char_p
    L.spa_last_error.argtypes = []
    L.spa_project.restype = st
    L.spa_project.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp]
    L.spa_attn_fwd_workspace_bytes.restype = z
    L.spa_attn_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.spa_attn_fwd_plan.restype = i
    L.spa_attn_fwd_plan.argtypes = [i, i, i, i, i, i, i, i]
    L.spa_attn_fwd.restype = st
    L.spa_attn_fwd.argtypes = [vp, vp, vp, vp, f, i, i, i, i, i, i, i, i, vp, i, vp, vp, z, vp]
    L.spa_attn_fwd_noalloc.restype = st
    L.spa_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, f, i, i, i, i, i, i, i, i, vp, i, vp, vp]
    L.spa_attn_fwd_noalloc_max_workspace_bytes.restype = z
    L.spa_attn_fwd_noalloc_max_workspace_bytes.argtypes = []
    L.spa_attn_bwd_workspace_bytes.restype = z
    L.spa_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.spa_attn_bwd.restype = st
    L.spa_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, f, i, i, i, i, i, i, i, i, vp, vp,
                               vp, vp, i, vp, z, vp]
    L.spa_sfa_fwd_workspace_bytes.restype = z
    L.spa_sfa_fwd_workspace_bytes.argtypes = [i, i, i, i, i]
    L.spa_sfa_fwd.restype = st
    L.spa_sfa_fwd.argtypes = [vp, vp, vp, i, f, i, i, i, i, i, i, i, vp, i, vp, vp, z, vp]
    L.spa_kcache_append.restype = st
    L.spa_kcache_append.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    L.spa_attn_decode_workspace_bytes.restype = z
    L.spa_attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    L.spa_attn_decode.restype = st
    L.spa_attn_decode.argtypes = [vp, vp, vp, vp, f, i, i, i, i, i, i, i, i, i, i, vp, i, vp,
                                  vp, z, vp]
    L.spa_profile_begin.restype = st
    L.spa_profile_begin.argtypes = [i]
    dp = ctypes.POINTER(ctypes.c_double)
    L.spa_profile_end.restype = st
    L.spa_profile_end.argtypes = [dp, dp, ctypes.POINTER(ctypes.c_int)]
    L.spa_probe_rates.restype = st
    L.spa_probe_rates.argtypes = [dp, dp, dp, dp, vp]
    _lib = L
    return L


def check(status: int) -> None:
    if status != SPA_OK:
        raise SpaError(status, lib().spa_last_error().decode())


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.bfloat16:
        return SPA_BF16
    if t == torch.float32:
        return SPA_F32
    raise TypeError(f"unsupported dtype {t}: use torch.bfloat16 or torch.float32")


def _device_tensor(x, name: str):
    if not x.is_cuda:
        raise ValueError(f"{name} must be a ROCm device tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x


def _same_device(ref, *others) -> None:
    """Every tensor (None skipped) must live on ref's device: the kernels run there."""
    for x in others:
        if x is not None and x.device != ref.device:
            raise ValueError(f"all tensors must be on {ref.device}; got one on {x.device}")


def _stream_ptr(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def spa_project(X, P):
    """Xt[b,h,n,:] = X[b,h,n,:] @ P[h] on the current stream. X [B,H,N,d], P [H,d,m]."""
    torch = _torch()
    _device_tensor(X, "X")
    _device_tensor(P, "P")
    if X.dim() != 4 or P.dim() != 3:
        raise ValueError("X must be [B,H,N,d] and P [H,d,m]")
    B, H, N, d = X.shape
    if P.shape[0] != H or P.shape[1] != d or P.dtype != X.dtype or P.device != X.device:
        raise ValueError("P must be [H,d,m] with X's dtype and device")
    m = P.shape[2]
    Xt = torch.empty((B, H, N, m), dtype=X.dtype, device=X.device)
    check(lib().spa_project(X.data_ptr(), P.data_ptr(), Xt.data_ptr(), B, H, N, d, m,
                            _dtype_code(X.dtype), _stream_ptr(X.device)))
    return Xt


def spa_attn_fwd_workspace_bytes(B, H, N, d, m, dv, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().spa_attn_fwd_workspace_bytes(B, H, N, d, m, dv, code))


def spa_attn_fwd_plan(B, H, N, d, m, dv, dtype, causal) -> int:
    """SPA_PLAN_* flags of how spa_attn_fwd runs these sizes (-1: unsupported)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().spa_attn_fwd_plan(B, H, N, d, m, dv, code, 1 if causal else 0))


def spa_attn_fwd(Q, K, V, P, scale: float | None = None, causal: bool = False,
                 out_dtype=None, return_lse: bool = False, workspace=None, out=None):
    """O = softmax(scale (Q P)(K P)^T [+causal]) V, per batch and head, on the current stream.

    Q, K [B,H,N,d], V [B,H,N,dv], P [H,d,m], all bf16 or all fp32 on one device.
    scale defaults to 1/sqrt(d). out_dtype: torch.float32 or torch.bfloat16 (bf16 inputs
    only); default is the input dtype. workspace: optional uint8 device tensor of at least
    spa_attn_fwd_workspace_bytes(...) bytes (otherwise the library allocates one
    stream-ordered). out: optional preallocated output. Returns O, or (O, lse) with lse the
    natural log of each row's softmax normaliser, fp32 [B,H,N].
    """
    torch = _torch()
    for name, x in (("Q", Q), ("K", K), ("V", V), ("P", P)):
        _device_tensor(x, name)
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError("Q, K must be [B,H,N,d] and V [B,H,N,dv]")
    B, H, N, d = Q.shape
    dv = V.shape[3]
    if P.dim() != 3 or P.shape[0] != H or P.shape[1] != d:
        raise ValueError("P must be [H,d,m]")
    m = P.shape[2]
    dt = Q.dtype
    if any(x.dtype != dt for x in (K, V, P)) or any(x.device != Q.device for x in (K, V, P)):
        raise ValueError("Q, K, V and P must share dtype and device")
    odt = dt if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=odt, device=Q.device)
    else:
        _device_tensor(out, "out")
        if out.shape != (B, H, N, dv) or out.dtype != odt:
            raise ValueError("out has the wrong shape or dtype")
    lse = torch.empty((B, H, N), dtype=torch.float32, device=Q.device) if return_lse else None
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _device_tensor(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _same_device(Q, out, workspace)
    check(lib().spa_attn_fwd(Q.data_ptr(), K.data_ptr(), V.data_ptr(), P.data_ptr(),
                             float(scale), int(bool(causal)), B, H, N, d, m, dv,
                             _dtype_code(dt), out.data_ptr(), _dtype_code(odt),
                             lse.data_ptr() if lse is not None else None, ws_ptr, ws_bytes,
                             _stream_ptr(Q.device)))
    return (out, lse) if return_lse else out


def spa_attn_fwd_noalloc(Q, K, V, P, scale: float | None = None, causal: bool = False,
                         out=None, out_dtype=None, lse=None):
    """spa_attn_fwd through the allocation-free entry point (the library's static workspace;
    the caller passes the outputs). Q, K, V, P as for spa_attn_fwd; out [B,H,N,dv] and the
    optional lse [B,H,N] fp32 are preallocated device tensors (created here if None, which is
    the binding's allocation, not the library's). Returns out."""
    torch = _torch()
    for name, x in (("Q", Q), ("K", K), ("V", V), ("P", P)):
        _device_tensor(x, name)
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError("Q, K must be [B,H,N,d] and V [B,H,N,dv]")
    B, H, N, d = Q.shape
    dv = V.shape[3]
    if P.dim() != 3 or P.shape[0] != H or P.shape[1] != d:
        raise ValueError("P must be [H,d,m]")
    m = P.shape[2]
    dt = Q.dtype
    if any(x.dtype != dt for x in (K, V, P)) or any(x.device != Q.device for x in (K, V, P)):
        raise ValueError("Q, K, V and P must share dtype and device")
    odt = out.dtype if out is not None else (dt if out_dtype is None else out_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=odt, device=Q.device)
    _device_tensor(out, "out")
    if out.shape != (B, H, N, dv):
        raise ValueError("out has the wrong shape")
    if lse is not None:
        _device_tensor(lse, "lse")
        if lse.shape != (B, H, N) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B,H,N]")
    _same_device(Q, out, lse)
    check(lib().spa_attn_fwd_noalloc(Q.data_ptr(), K.data_ptr(), V.data_ptr(), P.data_ptr(),
                                     float(scale), int(bool(causal)), B, H, N, d, m, dv,
                                     _dtype_code(dt), out.data_ptr(), _dtype_code(odt),
                                     lse.data_ptr() if lse is not None else None,
                                     _stream_ptr(Q.device)))
    return out


def spa_attn_fwd_noalloc_max_workspace_bytes() -> int:
    return int(lib().spa_attn_fwd_noalloc_max_workspace_bytes())


def spa_attn_bwd_workspace_bytes(B, H, N, d, m, dv, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(lib().spa_attn_bwd_workspace_bytes(B, H, N, d, m, dv, code))


def spa_attn_bwd(Q, K, V, P, O, dO, lse, scale: float | None = None, causal: bool = False,
                 grad_dtype=None, workspace=None):
    """Gradients (dQ, dK, dV, dP) of a loss through spa_attn_fwd, given dO = dL/dO.

    Q, K, V, P as passed to spa_attn_fwd (bf16, or float32 for the fp32 path); O the
    forward's output and lse its log-sum-exp (fp32 [B,H,N], spa_attn_fwd(...,
    return_lse=True)); O and dO in the inputs' dtype. grad_dtype: torch.float32 or
    torch.bfloat16 for dQ, dK, dV (default float32; float32 only on the fp32 path); dP is
    fp32 [H,d,m]. Runs on the current stream. On the bf16 path at m <= 64 the projected-query
    gradient is summed with fp32 atomic adds, so dQ and dP agree between runs to rounding and
    dK, dV bit for bit; the fp32 path is bit-for-bit deterministic.
    """
    torch = _torch()
    for name, x in (("Q", Q), ("K", K), ("V", V), ("P", P), ("O", O), ("dO", dO), ("lse", lse)):
        _device_tensor(x, name)
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError("Q, K must be [B,H,N,d] and V [B,H,N,dv]")
    B, H, N, d = Q.shape
    dv = V.shape[3]
    if P.dim() != 3 or P.shape[0] != H or P.shape[1] != d:
        raise ValueError("P must be [H,d,m]")
    m = P.shape[2]
    if O.shape != V.shape or dO.shape != V.shape or lse.shape != (B, H, N):
        raise ValueError("O and dO must be [B,H,N,dv] and lse [B,H,N]")
    if lse.dtype != torch.float32:
        raise ValueError("lse must be float32")
    dt = Q.dtype
    if any(x.dtype != dt for x in (K, V, P, O, dO)):
        raise ValueError("Q, K, V, P, O and dO must share a dtype")
    _same_device(Q, K, V, P, O, dO, lse, workspace)
    gdt = torch.float32 if grad_dtype is None else grad_dtype
    dQ = torch.empty((B, H, N, d), dtype=gdt, device=Q.device)
    dK = torch.empty((B, H, N, d), dtype=gdt, device=Q.device)
    dV = torch.empty((B, H, N, dv), dtype=gdt, device=Q.device)
    dP = torch.empty((H, d, m), dtype=torch.float32, device=Q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _device_tensor(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().spa_attn_bwd(Q.data_ptr(), K.data_ptr(), V.data_ptr(), P.data_ptr(),
                             O.data_ptr(), dO.data_ptr(), lse.data_ptr(), float(scale),
                             int(bool(causal)), B, H, N, d, m, dv, _dtype_code(dt),
                             dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), dP.data_ptr(),
                             _dtype_code(gdt), ws_ptr, ws_bytes, _stream_ptr(Q.device)))
    return dQ, dK, dV, dP


def spa_sfa_fwd_workspace_bytes(B, H, N, d, dv) -> int:
    return int(lib().spa_sfa_fwd_workspace_bytes(B, H, N, d, dv))


def spa_sfa_fwd(Q, K, V, topk: int, scale: float | None = None, causal: bool = False,
                out_dtype=None, return_lse: bool = False, workspace=None):
    """Sparse feature attention: softmax(scale Topk(Q) Topk(K)^T [+causal]) V on the
    current stream. Q, K [B,H,N,d] and V [B,H,N,dv] bf16; returns O [B,H,N,dv] (float32 by
    default, or out_dtype) and lse [B,H,N] if asked."""
    torch = _torch()
    for name, x in (("Q", Q), ("K", K), ("V", V)):
        _device_tensor(x, name)
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError("Q, K must be [B,H,N,d] and V [B,H,N,dv]")
    B, H, N, d = Q.shape
    dv = V.shape[3]
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("Q, K and V must share a dtype")
    _same_device(Q, K, V, workspace)
    odt = torch.float32 if out_dtype is None else out_dtype
    O = torch.empty((B, H, N, dv), dtype=odt, device=Q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=Q.device) if return_lse else None
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _device_tensor(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().spa_sfa_fwd(Q.data_ptr(), K.data_ptr(), V.data_ptr(), int(topk), float(scale),
                            int(bool(causal)), B, H, N, d, dv, _dtype_code(Q.dtype),
                            O.data_ptr(), _dtype_code(odt),
                            lse.data_ptr() if lse is not None else None, ws_ptr, ws_bytes,
                            _stream_ptr(Q.device)))
    return (O, lse) if return_lse else O


def spa_kcache_append(K, P, cache, row0: int) -> None:
    """cache[b,h,row0:row0+N,:] = fp16(K[b,h] @ P[h]) on the current stream.

    K [B,H,N,d] bf16 (the new keys), P [H,d,m] bf16, cache [B,H,rows,m] float16 (device,
    caller-owned, modified in place).
    """
    torch = _torch()
    for name, x in (("K", K), ("P", P), ("cache", cache)):
        _device_tensor(x, name)
    if K.dim() != 4 or P.dim() != 3 or cache.dim() != 4:
        raise ValueError("K must be [B,H,N,d], P [H,d,m] and cache [B,H,rows,m]")
    B, H, N, d = K.shape
    m = P.shape[2]
    if P.shape[:2] != (H, d) or cache.shape[:2] != (B, H) or cache.shape[3] != m:
        raise ValueError("P must be [H,d,m] and cache [B,H,rows,m]")
    if cache.dtype != torch.float16:
        raise ValueError("the key cache is float16")
    if K.dtype != P.dtype:
        raise ValueError("K and P must share a dtype")
    _same_device(K, P, cache)
    check(lib().spa_kcache_append(K.data_ptr(), P.data_ptr(), cache.data_ptr(), B, H, N, d, m,
                                  cache.shape[2], int(row0), _dtype_code(K.dtype),
                                  _stream_ptr(K.device)))


def spa_attn_decode_workspace_bytes(B, H, Nq, Nk, dv) -> int:
    return int(lib().spa_attn_decode_workspace_bytes(B, H, Nq, Nk, dv))


def spa_attn_decode(Q, cache, Vc, P, Nk: int, scale: float | None = None, causal: bool = True,
                    out_dtype=None, return_lse: bool = False, workspace=None):
    """Nq queries against the first Nk rows of a projected-key cache and a value cache.

    Q [B,H,Nq,d] bf16; cache [B,H,rows,m] float16 (spa_kcache_append); Vc [B,H,rows,dv]
    bf16; P [H,d,m] bf16. causal: query i sits at position Nk - Nq + i. Returns O
    [B,H,Nq,dv] (out_dtype float32 by default, or bfloat16), and lse if asked. Runs on the
    current stream.
    """
    torch = _torch()
    for name, x in (("Q", Q), ("cache", cache), ("Vc", Vc), ("P", P)):
        _device_tensor(x, name)
    if Q.dim() != 4 or cache.dim() != 4 or Vc.dim() != 4 or P.dim() != 3:
        raise ValueError("Q, cache, Vc must be 4-D and P [H,d,m]")
    B, H, Nq, d = Q.shape
    rows, m = cache.shape[2], cache.shape[3]
    dv = Vc.shape[3]
    if cache.shape[:2] != (B, H) or Vc.shape[:3] != (B, H, rows) or P.shape != (H, d, m):
        raise ValueError("cache [B,H,rows,m], Vc [B,H,rows,dv] and P [H,d,m] must agree")
    if cache.dtype != torch.float16:
        raise ValueError("the key cache is float16")
    if Q.dtype != Vc.dtype or Q.dtype != P.dtype:
        raise ValueError("Q, Vc and P must share a dtype")
    _same_device(Q, cache, Vc, P, workspace)
    odt = torch.float32 if out_dtype is None else out_dtype
    O = torch.empty((B, H, Nq, dv), dtype=odt, device=Q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=Q.device) if return_lse else None
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _device_tensor(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().spa_attn_decode(Q.data_ptr(), cache.data_ptr(), Vc.data_ptr(), P.data_ptr(),
                                float(scale), int(bool(causal)), B, H, Nq, int(Nk), rows, d, m,
                                dv, _dtype_code(Q.dtype), O.data_ptr(), _dtype_code(odt),
                                lse.data_ptr() if lse is not None else None, ws_ptr, ws_bytes,
                                _stream_ptr(Q.device)))
    return (O, lse) if return_lse else O


def profile_begin(max_calls: int) -> None:
    """Start recording per-launch HIP events for the next max_calls spa_attn_fwd calls."""
    check(lib().spa_profile_begin(int(max_calls)))


def probe_rates(device=None) -> dict:
    """Measured bf16 MFMA and fp32 VALU FMA rates (TFLOP/s) with the engine clock (GHz) while
    each ran, on the current stream (spa_probe_rates)."""
    torch = _torch()
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = [ctypes.c_double() for _ in range(4)]
    check(lib().spa_probe_rates(*(ctypes.byref(o) for o in out), _stream_ptr(dev)))
    return {"mfma_bf16_tflops": out[0].value, "mfma_clock_ghz": out[1].value,
            "fp32_fma_tflops": out[2].value, "fp32_clock_ghz": out[3].value}


def profile_end() -> tuple[float, float, int]:
    """(projection ms summed, attention ms summed, calls recorded); waits for the events."""
    p, a, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    check(lib().spa_profile_end(ctypes.byref(p), ctypes.byref(a), ctypes.byref(n)))
    return p.value, a.value, n.value


_attention_fn = None


def _attention_function():
    """The torch.autograd.Function over spa_attn_fwd / spa_attn_bwd (built on first use, so
    importing this module does not import torch)."""
    global _attention_fn
    if _attention_fn is not None:
        return _attention_fn
    torch = _torch()

    class SpaAttentionFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, Q, K, V, P, scale, causal):
            O, lse = spa_attn_fwd(Q, K, V, P, scale, causal, return_lse=True)
            ctx.save_for_backward(Q, K, V, P, O, lse)
            ctx.scale, ctx.causal = scale, causal
            return O

        @staticmethod
        def backward(ctx, dO):
            Q, K, V, P, O, lse = ctx.saved_tensors
            # autograd may hand over a strided view (the expanded ones of a plain sum); the
            # library reads dense rows
            dO = dO.contiguous()
            dQ, dK, dV, dP = spa_attn_bwd(Q, K, V, P, O, dO, lse, ctx.scale, ctx.causal,
                                          grad_dtype=Q.dtype)
            return dQ, dK, dV, dP, None, None

    _attention_fn = SpaAttentionFunction
    return _attention_fn


def spa_attention(Q, K, V, P, scale: float | None = None, causal: bool = False):
    """O = spa_attn_fwd(Q, K, V, P, scale, causal) recorded for autograd: the backward runs
    spa_attn_bwd from the saved inputs, output and log-sum-exp, so Q, K, V and the projection
    P (trained by its gradient as in SPA, Sec. 3.4.1 Gradient Flow and Algorithm 2) all
    receive gradients. dQ, dK and dV come out of the library in the inputs' dtype; dP comes
    out in fp32 and autograd casts it to P's dtype. O is in the inputs' dtype."""
    if scale is None:
        scale = 1.0 / math.sqrt(Q.shape[-1])
    return _attention_function().apply(Q, K, V, P, float(scale), bool(causal))
