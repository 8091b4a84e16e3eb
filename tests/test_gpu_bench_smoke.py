"""bench.py end to end on a short run: it prints one JSON line with the
contract's fields, the headline workload and operation, a roofline object
whose numbers agree with each other, and refuses more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, timeout=240):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_bench_prints_the_contract_line():
    r = run("--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-adapter",
            "--no-per-config", "--no-ceilings")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    j = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline"):
        assert k in j, k
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1
    assert j["unit"] == "GB/s" and j["higher_is_better"] is True
    assert j["config"]["workload"] == "cross-4096x11008-f16"
    assert j["value_op"]["op"] == "sddmm"
    rf = j["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert abs(j["value"] - rf["achieved"]) <= 0.01 * rf["achieved"] + 0.1
    # value = algorithmic bytes / the operation's time
    assert abs(j["value"] - j["value_op"]["alg_bytes"] / j["value_op"]["us"] / 1e3) \
        <= 0.01 * j["value"]
    assert 0 < j["value"] < 8000.0


def test_bench_refuses_several_gpus():
    r = run("--gpus", "2", timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr
