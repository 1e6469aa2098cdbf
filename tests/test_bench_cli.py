"""bench.py's command-line contract, on the CPU: one GPU only, and no GPU means no number."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line: nothing was measured


def test_world_size_above_one_is_refused():
    r = _run(env=dict(os.environ, WORLD_SIZE="8"))
    assert r.returncode == 2 and r.stdout.strip() == ""


def test_no_gpu_prints_no_number():
    import torch
    if torch.cuda.is_available():
        import pytest
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0 and r.stdout.strip() == ""
