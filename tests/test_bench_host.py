"""bench.py's host-side contract (no GPU needed): it measures one GPU only and says so for any
other count, and it refuses to run without a GPU instead of falling back to the CPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = _run("--gpus", n)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_no_gpu_means_no_result():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""
