"""ctypes wrapper for the double-precision CPU oracle (``spa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the benchmark's CPU
baseline leg are the only callers. The HIP library never imports or links this module, and
this module imports nothing from the HIP package.

Arrays are converted to C-contiguous float64; torch tensors (bf16 or fp32) convert exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspa_oracle.so")
SRC_PATH = os.path.join(_HERE, "spa_oracle.c")

_lib = None


def build(src: str = SRC_PATH, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (OpenMP, no fast-math: IEEE double order is kept)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    _lib = configure(ctypes.CDLL(LIB_PATH))
    return _lib


def configure(lib):
    """Declare the C signatures on a loaded copy of the oracle library."""
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.spa_oracle_threads.argtypes = [ctypes.c_int]
    lib.spa_oracle_threads.restype = ctypes.c_int
    lib.spa_oracle_project.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, ctypes.c_int]
    lib.spa_oracle_project.restype = ctypes.c_int
    lib.spa_oracle_attn_fwd.argtypes = [dp, dp, dp, dp, ctypes.c_double, ctypes.c_int,
                                        i64, i64, i64, i64, i64, i64, dp, dp, ctypes.c_int]
    lib.spa_oracle_attn_fwd.restype = ctypes.c_int
    lib.spa_oracle_attn_rows.argtypes = [dp, dp, dp, dp, ctypes.c_double, ctypes.c_int,
                                         i64, i64, i64, i64, i64, i64, ip, ip, i64, dp, dp,
                                         ctypes.c_int]
    lib.spa_oracle_attn_rows.restype = ctypes.c_int
    lib.spa_oracle_attn_bwd.argtypes = [dp, dp, dp, dp, dp, ctypes.c_double, ctypes.c_int,
                                        i64, i64, i64, i64, i64, i64, dp, dp, dp, dp,
                                        ctypes.c_int]
    lib.spa_oracle_attn_bwd.restype = ctypes.c_int
    for name in ("spa_oracle_scores", "spa_oracle_weights"):
        f = getattr(lib, name)
        f.argtypes = [dp, dp, dp, ctypes.c_double, ctypes.c_int, i64, i64, i64, i64, i64, dp,
                      ctypes.c_int]
        f.restype = ctypes.c_int
    return lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: exact widening on the CPU
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def threads(nthreads: int = 0) -> int:
    """Threads the oracle uses for a request (0 = every available core)."""
    return int(_load().spa_oracle_threads(nthreads))


def _shape4(Q, K, V, P):
    if Q.ndim != 4 or K.shape != Q.shape or V.ndim != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError("Q, K must be [B,H,N,d] and V [B,H,N,dv]")
    B, H, N, d = Q.shape
    if P.shape[0] != H or P.shape[1] != d:
        raise ValueError("P must be [H,d,m]")
    return B, H, N, d, P.shape[2], V.shape[3]


def project(X, P, nthreads: int = 0) -> np.ndarray:
    """Xt[b,h,n,:] = X[b,h,n,:] @ P[h]; X [B,H,N,d], P [H,d,m] -> [B,H,N,m]."""
    X, P = _f64(X), _f64(P)
    B, H, N, d = X.shape
    m = P.shape[2]
    out = np.empty((B, H, N, m))
    _check(_load().spa_oracle_project(_ptr(X), _ptr(P), _ptr(out), B, H, N, d, m, nthreads),
           "project")
    return out


def attn_fwd(Q, K, V, P, scale: float, causal: bool, with_lse: bool = False,
             nthreads: int = 0):
    """O = softmax(scale (Q P)(K P)^T [+causal mask]) V per head; returns O (and lse)."""
    Q, K, V, P = _f64(Q), _f64(K), _f64(V), _f64(P)
    B, H, N, d, m, dv = _shape4(Q, K, V, P)
    O = np.empty((B, H, N, dv))
    lse = np.empty((B, H, N)) if with_lse else None
    rc = _load().spa_oracle_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(P), float(scale),
                                     int(bool(causal)), B, H, N, d, m, dv, _ptr(O),
                                     _ptr(lse) if with_lse else None, nthreads)
    _check(rc, "attn_fwd")
    return (O, lse) if with_lse else O


def attn_bwd(Q, K, V, P, dO, scale: float, causal: bool, nthreads: int = 0):
    """Gradients of L = sum(dO * O) for the forward above: (dQ, dK, dV, dP), float64."""
    Q, K, V, P, dO = _f64(Q), _f64(K), _f64(V), _f64(P), _f64(dO)
    B, H, N, d, m, dv = _shape4(Q, K, V, P)
    if dO.shape != V.shape:
        raise ValueError("dO must have the shape of V (and of O)")
    dQ, dK = np.empty((B, H, N, d)), np.empty((B, H, N, d))
    dV, dP = np.empty((B, H, N, dv)), np.empty((H, d, m))
    rc = _load().spa_oracle_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(P), _ptr(dO), float(scale),
                                     int(bool(causal)), B, H, N, d, m, dv, _ptr(dQ), _ptr(dK),
                                     _ptr(dV), _ptr(dP), nthreads)
    _check(rc, "attn_bwd")
    return dQ, dK, dV, dP


def attn_rows(Q, K, V, P, scale: float, causal: bool, row_bh, row_i, with_lse: bool = False,
              nthreads: int = 0):
    """Forward on sampled rows: output k is query row_i[k] of flattened head row_bh[k]."""
    Q, K, V, P = _f64(Q), _f64(K), _f64(V), _f64(P)
    B, H, N, d, m, dv = _shape4(Q, K, V, P)
    rb = np.ascontiguousarray(row_bh, dtype=np.int64)
    ri = np.ascontiguousarray(row_i, dtype=np.int64)
    if rb.shape != ri.shape or rb.ndim != 1:
        raise ValueError("row_bh and row_i must be 1-D and of equal length")
    n = rb.shape[0]
    O = np.empty((n, dv))
    lse = np.empty(n) if with_lse else None
    ip = ctypes.POINTER(ctypes.c_int64)
    rc = _load().spa_oracle_attn_rows(_ptr(Q), _ptr(K), _ptr(V), _ptr(P), float(scale),
                                      int(bool(causal)), B, H, N, d, m, dv,
                                      rb.ctypes.data_as(ip), ri.ctypes.data_as(ip), n,
                                      _ptr(O), _ptr(lse) if with_lse else None, nthreads)
    _check(rc, "attn_rows")
    return (O, lse) if with_lse else O


def attn_decode(Q, K, V, P, scale: float, causal: bool, with_lse: bool = False,
                nthreads: int = 0):
    """Nq queries against Nk keys, Q [B,H,Nq,d], K [B,H,Nk,d], V [B,H,Nk,dv], Nq <= Nk.

    Reading of a rectangular causal mask (no page defines one): the queries are the last Nq
    positions of the sequence, query i at position Nk - Nq + i, seeing keys j <= Nk - Nq + i,
    so the result is rows Nk - Nq .. Nk - 1 of the square forward above. Computed that way:
    the queries are placed in those rows of an otherwise zero [B,H,Nk,d] query tensor and
    only those rows are evaluated (attn_rows). Returns O [B,H,Nq,dv] (and lse [B,H,Nq]).
    """
    Q, K = _f64(Q), _f64(K)
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    if K.shape[:2] != (B, H) or K.shape[3] != d or Nq > Nk:
        raise ValueError("Q [B,H,Nq,d] and K [B,H,Nk,d] with Nq <= Nk")
    Qfull = np.zeros((B, H, Nk, d))
    Qfull[:, :, Nk - Nq:] = Q
    rb = np.repeat(np.arange(B * H, dtype=np.int64), Nq)
    ri = np.tile(np.arange(Nk - Nq, Nk, dtype=np.int64), B * H)
    out = attn_rows(Qfull, K, V, P, scale, causal, rb, ri, with_lse=with_lse,
                    nthreads=nthreads)
    dv = _f64(V).shape[3]
    if with_lse:
        return out[0].reshape(B, H, Nq, dv), out[1].reshape(B, H, Nq)
    return out.reshape(B, H, Nq, dv)


def topk_features(X, k: int) -> np.ndarray:
    """Row-wise Top-k along the last axis (Scaling Attention via Feature Sparsity, key design
    1): keep x_u where u is among the k coordinates of largest |x|, zero elsewhere. Reading
    for ties in |x| (the page does not break them): the lower coordinate index wins."""
    X = _f64(X)
    d = X.shape[-1]
    if not 1 <= k <= d:
        raise ValueError("k must be in [1, d]")
    # a stable sort by -|x| keeps equal magnitudes in index order
    keep = np.argsort(-np.abs(X), axis=-1, kind="stable")[..., :k]
    out = np.zeros_like(X)
    np.put_along_axis(out, keep, np.take_along_axis(X, keep, axis=-1), axis=-1)
    return out


def sfa_fwd(Q, K, V, k: int, scale: float, causal: bool, with_lse: bool = False,
            nthreads: int = 0):
    """Sparse feature attention: softmax(scale Topk_k(Q) Topk_k(K)^T [+causal]) V, exact,
    computed as the forward above with P = I on the Top-k rows."""
    Qs, Ks = topk_features(Q, k), topk_features(K, k)
    H, d = Qs.shape[1], Qs.shape[3]
    eye = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    return attn_fwd(Qs, Ks, V, eye, scale, causal, with_lse=with_lse, nthreads=nthreads)


def _matrix(fn_name: str, Q, K, P, scale: float, causal: bool, nthreads: int) -> np.ndarray:
    Q, K, P = _f64(Q), _f64(K), _f64(P)
    B, H, N, d = Q.shape
    if K.shape != Q.shape or P.shape[:2] != (H, d):
        raise ValueError("Q, K must be [B,H,N,d] and P [H,d,m]")
    out = np.empty((B, H, N, N))
    rc = getattr(_load(), fn_name)(_ptr(Q), _ptr(K), _ptr(P), float(scale),
                                   int(bool(causal)), B, H, N, d, P.shape[2], _ptr(out),
                                   nthreads)
    _check(rc, fn_name)
    return out


def scores(Q, K, P, scale: float, causal: bool, nthreads: int = 0) -> np.ndarray:
    """Projected scores scale (Q P)(K P)^T per head, -inf where the causal mask applies."""
    return _matrix("spa_oracle_scores", Q, K, P, scale, causal, nthreads)


def weights(Q, K, P, scale: float, causal: bool, nthreads: int = 0) -> np.ndarray:
    """Row-softmax attention weights of the projected scores (masked entries are 0)."""
    return _matrix("spa_oracle_weights", Q, K, P, scale, causal, nthreads)
