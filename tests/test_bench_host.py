"""Host-side checks of bench.py and the binding that need no GPU: the bench
refuses more than one GPU, and neither the bench nor the binding falls back
to the CPU when no GPU is present."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_bench_refuses_more_than_one_gpu():
    r = run_bench("--gpus", "2")
    assert r.returncode != 0
    assert "--gpus 1" in r.stdout + r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour without a GPU")
def test_bench_fails_without_a_gpu():
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "needs a GPU" in r.stdout + r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour without a GPU")
def test_binding_rejects_host_tensors():
    from linear_attention_long_amd import api
    q = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError, match="GPU"):
        api.la_prefill(q, q, q)
