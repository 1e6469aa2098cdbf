"""bench.py's JSON line on a GPU: the keys and units the benchmark contract asks for, a
roofline object consistent with its own figures, and the oracle's CPU baseline beside it.
Runs the real benchmark briefly (few steps, a short CPU sample) in a child process."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def line():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench line: bench.py --steps 3 --warmup 1 --cpu-budget 2", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--cpu-budget", "2"], cwd=ROOT, capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, f"expected one JSON line, got {len(lines)}"
    return json.loads(lines[0])


def test_contract_keys(line):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["warmup"] == 1
    assert line["unit"] == "blocks/s" and line["higher_is_better"] is True
    assert line["dtype"] == "bf16" and line["vs_baseline"] is None
    assert line["value"] > 0 and line["ms_per_step"] > 0
    assert "workload" in line["config"] and line["config"]["B"] == 32 and line["config"]["S"] == 16


def test_value_is_blocks_per_second_of_the_attention_call(line):
    # value = B / t_attn, with t_attn the back-to-back attention call
    assert line["value"] == pytest.approx(line["config"]["B"] / (line["attn_us_per_call"] * 1e-6), rel=1e-9)


def test_roofline_object(line):
    rf = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    # achieved = algorithmic bytes per launch / the main kernel's average duration
    assert rf["achieved"] == pytest.approx(rf["algorithmic_bytes_per_launch"] / (rf["avg_us"] * 1e-6) / 1e9,
                                           rel=1e-9)
    assert 0 < rf["frac"] < 1
    assert rf["traffic"] is None or rf["traffic"] >= rf["algorithmic_bytes_per_launch"]


def test_cpu_baseline(line):
    cb = line["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cb, k
    assert cb["kind"] == "oracle" and cb["unit"] == "blocks/s" and cb["value"] > 0 and cb["cores"] >= 1
