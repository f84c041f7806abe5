"""CPU checks of bench.py's command-line contract (no GPU needed)."""
import os
import subprocess
import sys

from conftest import ROOT


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no result line


def test_fails_loudly_without_a_usable_gpu():
    """Where no gfx950 device is visible the bench must stop with an error,
    never print a result line from some other path."""
    import torch
    if torch.cuda.is_available():
        import pytest
        pytest.skip("a GPU is visible")
    r = run_bench("--quick", "--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0
    assert not any(line.startswith("{") for line in r.stdout.splitlines())
