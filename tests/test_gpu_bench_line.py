"""The benchmark's JSON line on the GPU: a short run (two timed rounds, no
oracle leg, no other configurations or secondary figures) prints one line
that carries every field of the contract, with a roofline entry for the
dominant kernel whose figures agree with each other."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_short_bench_run_prints_one_contract_line():
    print("[bench] --steps 2 --warmup 1 --rounds 2 --no-cpu --no-configs --no-secondary", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1", "--rounds",
                        "2", "--no-cpu", "--no-configs", "--no-secondary"], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    line = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 2 and line["warmup"] == 1
    assert line["higher_is_better"] is True and line["vs_baseline"] is None
    assert line["config"]["workload"] and line["config"]["B"] == 256 and line["config"]["gamma"] == 5
    # drafted positions per second from the step time
    assert abs(line["value"] - 256 * 5 / (line["ms_per_step"] * 1e-3)) <= 1e-3 * line["value"]
    rf = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0.0 < rf["frac"] < 1.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) <= 1e-3
