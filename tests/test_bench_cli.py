"""The benchmark's command line (CPU): the refusals that come before any GPU work."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_query_count_is_checked_first():
    r = run("--decode", "--decode-queries", "0")
    assert r.returncode == 2
    assert "--decode-queries" in r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the refusal without a GPU")
def test_without_a_gpu_the_benchmark_refuses():
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a ROCm GPU" in r.stderr
