"""Algorithmic work and traffic of the projected-attention forward and backward (host-side
arithmetic).

Work per head, following the cost model of the Sparse Projection Attention page (Sec. 4.1.1,
dense projection, s = 1) and the time-complexity list of the Projection-Decomposition
Attention page (Sec. 4.1, steps 1-3 and 5 without the low-rank step):

    project Q and K : 2 * (2 N d m)        = 4 N d m
    scores          : c * 2 N^2 m
    weights x V     : c * 2 N^2 dv
    exponentials    : c * N^2

with c = 1/2 under a causal mask (the N^2 terms are halved; the projection term is not).

Bytes per head of the whole path: read Q, K, V and P once, write O once, and one round trip
(write plus read) of the projected keys and queries that the projection launch hands to the
attention launch. Where the attention launch projects the queries itself, only the keys make
that round trip, and the queries (and P) are read by the attention launch. The exact-score
work the method avoids is never counted.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Work:
    project_flops: float
    score_flops: float
    pv_flops: float
    exps: float

    @property
    def attn_flops(self) -> float:
        """Flops of the attention launch (scores and weights x V)."""
        return self.score_flops + self.pv_flops

    @property
    def total_flops(self) -> float:
        return self.project_flops + self.score_flops + self.pv_flops


def work(B: int, H: int, N: int, d: int, m: int, dv: int, causal: bool) -> Work:
    heads = B * H
    c = 0.5 if causal else 1.0
    return Work(project_flops=heads * 4.0 * N * d * m,
                score_flops=heads * c * 2.0 * N * N * m,
                pv_flops=heads * c * 2.0 * N * N * dv,
                exps=heads * c * float(N) * N)


@dataclass(frozen=True)
class BwdWork:
    """Backward work: the five N^2 contractions of the chain rule (scores recomputed, dA,
    dV, dQt, dKt) and the projection-side products (Qt, Kt recomputed, dQ, dK, dP)."""

    n2_flops: float          # c N^2 (6m + 4dv) per head
    projection_flops: float  # 12 N d m per head
    executed_n2_flops: float  # what the kernels run: scores and dA are formed twice

    @property
    def total_flops(self) -> float:
        return self.n2_flops + self.projection_flops


def bwd_work(B: int, H: int, N: int, d: int, m: int, dv: int, causal: bool) -> BwdWork:
    c = 0.5 if causal else 1.0
    heads = B * H
    return BwdWork(
        n2_flops=heads * c * N * N * (6.0 * m + 4.0 * dv),
        projection_flops=heads * 12.0 * N * d * m,
        executed_n2_flops=heads * c * N * N * (8.0 * m + 6.0 * dv),
    )


def path_bytes(B: int, H: int, N: int, d: int, m: int, dv: int, elem: int = 2,
               out_elem: int = 2, queries_in_attention: bool = False) -> dict[str, float]:
    """Algorithmic HBM bytes of each launch and of the whole path (see module docstring)."""
    heads = B * H
    x = 1.0 * heads * N * d * elem  # Q or K
    v = 1.0 * heads * N * dv * elem
    o = 1.0 * heads * N * dv * out_elem
    p = 1.0 * H * d * m * elem
    tilde = 1.0 * heads * N * m * elem  # projected queries or keys
    if queries_in_attention:
        project = x + p + tilde  # read K, P; write Kt
        attn = x + p + tilde + v + o  # read Q, P, Kt, V; write O
    else:
        project = 2 * x + p + 2 * tilde  # read Q, K, P; write Qt, Kt
        attn = 2 * tilde + v + o  # read Qt, Kt, V; write O
    return {"project": project, "attn": attn, "total": project + attn}


def score_speedup(d: int, m: int) -> float:
    """Score-computation ratio of exact to projected attention, d/m (SPA page Sec. 3.1.3)."""
    return d / m


def asymptotic_speedup(d: int, m: int, dv: int) -> float:
    """End-to-end ratio as N grows, (d + dv)/(m + dv) (SPA page Sec. 4.1.1)."""
    return (d + dv) / (m + dv)


def materialised_logits_bytes(N: int, bytes_per_logit: int = 4) -> int:
    """Bytes of one head's N x N logit matrix, which this path never writes."""
    return N * N * bytes_per_logit


# MI355X published peaks used as roofline denominators.
PEAK_BF16_DENSE_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_FP32_VECTOR_TFLOPS = 157.3  # 256 CU x 2.4 GHz x 256 flop/clk/CU (128 fp32 FMA lanes)
PEAK_HBM_GBS = 8000.0
