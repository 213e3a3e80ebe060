"""Host-side work accounting against the pages' printed cost figures (no GPU)."""
import json
import math
import os

import pytest

from jl_feature_projected_amd import accounting, inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_cost_figures.json")


def _entries():
    with open(GOLDEN) as f:
        return json.load(f)["entries"]


def test_spa_cost_model_figures():
    e = _entries()[0]
    assert accounting.score_speedup(e["d"], e["m"]) == e["score_speedup"]
    # the asymptotic formula; the page rounds its value to "about 1.9"
    s = accounting.asymptotic_speedup(e["d"], e["m"], e["dv"])
    assert s == pytest.approx(1024 / 576)
    assert abs(s - e["end_to_end_speedup_printed"]) < 0.15
    # the work model reproduces the same limit as N grows
    N = 1 << 20
    proj = accounting.work(1, 1, N, e["d"], e["m"], e["dv"], False)
    exact = accounting.work(1, 1, N, e["d"], e["d"], e["dv"], False)
    ratio = (exact.score_flops + exact.pv_flops) / proj.total_flops
    assert ratio == pytest.approx(s, rel=1e-3)


def test_linformer_logit_memory_figure():
    e = _entries()[1]
    b = accounting.materialised_logits_bytes(e["N"], e["bytes_per_logit"])
    assert round(b / 1e6) == e["megabytes_printed"]


def test_work_formula_and_headline_numbers():
    w = inputs.WORKLOADS["c3"]
    k = accounting.work(w.B, w.H, w.N, w.d, w.m, w.dv, w.causal)
    heads = w.B * w.H
    assert k.project_flops == heads * 4 * w.N * w.d * w.m
    assert k.score_flops == heads * 0.5 * 2 * w.N ** 2 * w.m
    assert k.pv_flops == heads * 0.5 * 2 * w.N ** 2 * w.dv
    assert k.total_flops / 1e9 == pytest.approx(347.89, abs=0.01)
    # the time at the bf16 dense MFMA peak
    t_us = k.total_flops / (accounting.PEAK_BF16_DENSE_TFLOPS * 1e12) * 1e6
    assert t_us == pytest.approx(138.2, abs=0.1)
    # c5 sweep totals
    for m, gf in ((8, 585.19), (16, 620.62), (32, 691.49), (64, 833.22), (128, 1116.69)):
        x = inputs.WORKLOADS[f"c5_m{m}"]
        assert accounting.work(x.B, x.H, x.N, x.d, x.m, x.dv, True).total_flops / 1e9 == \
            pytest.approx(gf, abs=0.01)


def test_path_bytes():
    b = accounting.path_bytes(2, 16, 8192, 128, 32, 128)
    heads = 32
    assert b["project"] == 2 * heads * 8192 * 128 * 2 + 16 * 128 * 32 * 2 + 2 * heads * 8192 * 32 * 2
    assert b["attn"] == 2 * heads * 8192 * 32 * 2 + 2 * heads * 8192 * 128 * 2
    assert math.isclose(b["total"], b["project"] + b["attn"])
    # queries projected inside the attention launch: only the keys make the round trip
    f = accounting.path_bytes(2, 16, 8192, 128, 32, 128, queries_in_attention=True)
    x, p, t = heads * 8192 * 128 * 2, 16 * 128 * 32 * 2, heads * 8192 * 32 * 2
    assert f["project"] == x + p + t
    assert f["attn"] == x + p + t + 2 * heads * 8192 * 128 * 2
    assert math.isclose(b["total"] - f["total"], 2 * t - p)
