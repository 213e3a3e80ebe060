"""Seeded synthetic inputs for feature-axis projected softmax attention.

This module is shared by the CPU oracle's tests and by the HIP path's tests, smoke check and
benchmark. It draws random numbers and lays them out; it holds none of the attention
arithmetic. The Gaussian projection P that the method draws is drawn here and handed to both
sides as an input (Sparse Projection Attention, Sec. 2.1 Theorem 1 proof step 1 and
Projection-Decomposition Attention, Algorithm 2.1 step 1: entries iid N(0, 1/m)).

Recipe (one numpy PCG64 generator per workload, float64 throughout):
  1. P: for h in 0..H-1, P[h] = standard_normal((d, m)) / sqrt(m); or the identity when
     ``proj == "identity"`` (then m == d).
  2. for b in 0..B-1, for h in 0..H-1, in this order: Q block, K block, V block.
     * ``qk == "iid"``: standard_normal((N, d)).
     * ``qk == "lowrank"``: (A @ F) / sqrt(r) + 0.1 * E with A ~ (N, r), F ~ (r, d),
       E ~ (N, d), all standard normal, r = 16, drawn in the order A, F, E.
     * V: standard_normal((N, dv)).
     * Q and K rows are rescaled to L2 norm sqrt(d); V rows to sqrt(dv) when ``v_norm``.
  3. Storage rounding: float64 -> float32 (round to nearest even); for bf16 storage the float32
     value is then rounded to bf16 (round to nearest even, via torch on the CPU). The identical
     stored bits go to the GPU and, converted exactly to float64, to the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator

import numpy as np
import torch

LOWRANK_RANK = 16
LOWRANK_NOISE = 0.1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload: shapes, mask, storage dtype and input recipe."""

    name: str
    B: int
    H: int
    N: int
    d: int
    m: int
    dv: int
    causal: bool
    dtype: str = "bf16"  # storage and compute-input dtype: "bf16" or "f32"
    qk: str = "iid"  # "iid" or "lowrank"
    qk_norm: bool = True  # rescale Q and K rows to norm sqrt(d)
    v_norm: bool = True  # rescale V rows to norm sqrt(dv)
    proj: str = "gauss"  # "gauss" (N(0, 1/m)), "identity" (m == d), "sparse", "block", "banded"
    proj_s: float = 0.0  # "sparse": the sparsity level s (0: sqrt(d))
    proj_block: tuple = (16, 4)  # "block": a input features x b outputs per block
    proj_band: int = 16  # "banded": nonzeros per input feature
    seed: int = 0

    @property
    def scale(self) -> float:
        """Score scale 1/sqrt(d): keeps projected scores on the exact-score scale."""
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the benchmark and the parity tests use.
C5_M = (8, 16, 32, 64, 128)

WORKLOADS: dict[str, Workload] = {
    # one head, fp32, non-causal, all rows normalised
    "c1": Workload("single-head-n512-d64-m16-fp32", 1, 1, 512, 64, 16, 64, False,
                   dtype="f32", seed=101),
    # GPT-2-124M attention shape at length 2048, causal
    "c2": Workload("b4h12-n2048-d64-m16-causal", 4, 12, 2048, 64, 16, 64, True, seed=202),
    # low-rank-plus-noise Q/K, causal, V not normalised
    "c3": Workload("b2h16-n8192-d128-m32-causal-lowrank", 2, 16, 8192, 128, 32, 128, True,
                   qk="lowrank", v_norm=False, seed=303),
    # long-range classification shape, non-causal
    "c4": Workload("b1h32-n32768-d128-m16-noncausal", 1, 32, 32768, 128, 16, 128, False,
                   seed=404),
}
for _i, _m in enumerate(C5_M):
    WORKLOADS[f"c5_m{_m}"] = Workload(f"b1h16-n16384-d128-m{_m}-causal", 1, 16, 16384, 128,
                                      _m, 128, True, seed=505 + _i)
WORKLOADS["c5_identity"] = Workload("b1h16-n16384-d128-m128-identity-causal", 1, 16, 16384,
                                    128, 128, 128, True, proj="identity", seed=505 + len(C5_M))

# The headline workload: N=8192, d=128, m=32, causal.
HEADLINE = "c3"


def _rescale_rows(x: np.ndarray, norm: float) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    n[n == 0.0] = 1.0
    return x * (norm / n)


def _qk_block(rng: np.random.Generator, w: Workload) -> np.ndarray:
    if w.qk == "iid":
        x = rng.standard_normal((w.N, w.d))
    elif w.qk == "lowrank":
        a = rng.standard_normal((w.N, LOWRANK_RANK))
        f = rng.standard_normal((LOWRANK_RANK, w.d))
        e = rng.standard_normal((w.N, w.d))
        x = (a @ f) / math.sqrt(LOWRANK_RANK) + LOWRANK_NOISE * e
    else:
        raise ValueError(f"unknown qk recipe {w.qk!r}")
    if w.qk_norm:
        x = _rescale_rows(x, math.sqrt(w.d))
    return x


def sparse_projection(rng: np.random.Generator, d: int, m: int, s: float) -> np.ndarray:
    """[d, m]: the sparse random matrix of the Sparse Projection Attention page, Sec. 2.2
    Definition 1 -- each entry independently sqrt(s/m) times +1 or -1 with probability
    1/(2s) each, else 0 (s >= 1)."""
    if s < 1.0:
        raise ValueError("the sparsity level s must be >= 1")
    u = rng.random((d, m))
    sign = np.where(u < 0.5 / s, 1.0, np.where(u < 1.0 / s, -1.0, 0.0))
    return sign * math.sqrt(s / m)


def block_projection(rng: np.random.Generator, d: int, m: int, a: int, b: int) -> np.ndarray:
    """[d, m]: block pattern a x b -- input features [a r, a r + a) feed outputs
    [b c, b c + b) with c = r mod (m / b), entries N(0, 1/b) inside the blocks, zero
    elsewhere (every input feature has b nonzeros, so E[P P^T] = I)."""
    if d % a or m % b:
        raise ValueError("the block shape must divide d x m")
    p = np.zeros((d, m))
    for r in range(d // a):
        c = r % (m // b)
        p[a * r:a * r + a, b * c:b * c + b] = rng.standard_normal((a, b)) / math.sqrt(b)
    return p


def banded_projection(rng: np.random.Generator, d: int, m: int, w: int) -> np.ndarray:
    """[d, m]: banded pattern of width w -- input feature i feeds the w outputs
    (floor(i m / d) - w // 2 + t) mod m, t < w, with N(0, 1/w) entries (E[P P^T] = I)."""
    if not 1 <= w <= m:
        raise ValueError("the band width must be in [1, m]")
    p = np.zeros((d, m))
    for i in range(d):
        cols = (i * m // d - w // 2 + np.arange(w)) % m
        p[i, cols] = rng.standard_normal(w) / math.sqrt(w)
    return p


def _projection(rng: np.random.Generator, w: Workload) -> np.ndarray:
    if w.proj == "identity":
        if w.m != w.d:
            raise ValueError("identity projection needs m == d")
        return np.broadcast_to(np.eye(w.d), (w.H, w.d, w.d)).copy()
    p = np.empty((w.H, w.d, w.m))
    for h in range(w.H):
        if w.proj == "gauss":
            p[h] = rng.standard_normal((w.d, w.m)) / math.sqrt(w.m)
        elif w.proj == "sparse":
            p[h] = sparse_projection(rng, w.d, w.m, w.proj_s or math.sqrt(w.d))
        elif w.proj == "block":
            p[h] = block_projection(rng, w.d, w.m, *w.proj_block)
        elif w.proj == "banded":
            p[h] = banded_projection(rng, w.d, w.m, w.proj_band)
        else:
            raise ValueError(f"unknown projection {w.proj!r}")
    return p


def iter_f64(w: Workload) -> Iterator[tuple[str, tuple, np.ndarray]]:
    """Yield ("P", (), P[H,d,m]) then ("Q"|"K"|"V", (b, h), block) in draw order, float64."""
    rng = np.random.default_rng(w.seed)
    yield "P", (), _projection(rng, w)
    for b in range(w.B):
        for h in range(w.H):
            yield "Q", (b, h), _qk_block(rng, w)
            yield "K", (b, h), _qk_block(rng, w)
            v = rng.standard_normal((w.N, w.dv))
            if w.v_norm:
                v = _rescale_rows(v, math.sqrt(w.dv))
            yield "V", (b, h), v


def to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 -> float32 (RNE) -> bf16 (RNE) when dtype == "bf16"."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@dataclasses.dataclass
class Inputs:
    """Stored inputs (CPU tensors in the storage dtype), contiguous row-major.

    Q, K: [B, H, N, d]; V: [B, H, N, dv]; P: [H, d, m].
    """

    w: Workload
    Q: torch.Tensor
    K: torch.Tensor
    V: torch.Tensor
    P: torch.Tensor

    def f64(self, name: str) -> np.ndarray:
        """Exact float64 copy of a stored tensor (bf16 and fp32 convert exactly)."""
        return getattr(self, name).to(torch.float64).numpy()


def draw(w: Workload) -> Inputs:
    """Draw the stored inputs of a workload (CPU tensors in the storage dtype)."""
    dt = w.torch_dtype
    Q = torch.empty((w.B, w.H, w.N, w.d), dtype=dt)
    K = torch.empty((w.B, w.H, w.N, w.d), dtype=dt)
    V = torch.empty((w.B, w.H, w.N, w.dv), dtype=dt)
    P = None
    for name, idx, blk in iter_f64(w):
        if name == "P":
            P = to_storage(blk, w.dtype)
        else:
            {"Q": Q, "K": K, "V": V}[name][idx].copy_(to_storage(blk, w.dtype))
    return Inputs(w, Q, K, V, P)


def draw_f64(w: Workload) -> dict[str, np.ndarray]:
    """Pre-rounding float64 inputs of a (small) workload: P[H,d,m], Q, K [B,H,N,d], V."""
    out = {"Q": np.empty((w.B, w.H, w.N, w.d)), "K": np.empty((w.B, w.H, w.N, w.d)),
           "V": np.empty((w.B, w.H, w.N, w.dv))}
    for name, idx, blk in iter_f64(w):
        if name == "P":
            out["P"] = blk
        else:
            out[name][idx] = blk
    return out


def gaussian_projection(d: int, m: int, seed: int, heads: int = 1) -> np.ndarray:
    """P[heads, d, m] with iid N(0, 1/m) entries from its own PCG64 stream (float64)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((heads, d, m)) / math.sqrt(m)


def draw_grad_output(w: Workload, seed: int) -> torch.Tensor:
    """A seeded stand-in for dL/dO: iid N(0, 1) entries [B, H, N, dv] from its own PCG64
    stream, stored like the other inputs (float64 -> float32 -> bf16 RNE)."""
    rng = np.random.default_rng(seed)
    return to_storage(rng.standard_normal((w.B, w.H, w.N, w.dv)), w.dtype)
