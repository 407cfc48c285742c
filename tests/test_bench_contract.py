"""The benchmark's host-side contract, on the CPU: the one-GPU guard, the
algorithmic byte counts the roofline figures divide by, and the per-round
outcome counts the logit passes' bytes come from."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_draft_step_bytes_at_the_headline_size():
    b = _bench()
    B, V, r = 256, 129280, 256
    # U_k rows (float32), W2 (bf16) once, the gathered W1 rows (bf16)
    assert b._draft_bytes(B, V, r, 2) == B * V * 4 + V * r * 2 + B * r * 2
    assert round(b._draft_bytes(B, V, r, 2) / 1e6, 1) == 198.7


def test_logit_pass_bytes_and_fractions():
    b = _bench()
    V, r = 129280, 256
    row = V * 4
    phases = {"verify_walk": {"avg_us": 50.0}, "verify_tail": {"avg_us": 20.0}, "verify_draw": {"avg_us": 40.0}}
    outcome = {"rows": 500.0, "residual": 200.0, "bonus": 30.0}
    out = b._logit_passes(phases, outcome, 256, V, r)
    walk = out["verify_walk"]
    assert walk["bytes"] == int(500 * row) and walk["us"] == 70.0  # the tail's time counts with the walk
    assert walk["frac"] == round(500 * row / 70e-6 / 1e9 / b.HBM_PEAK_GBS, 4)
    draw = out["verify_draw"]
    assert draw["bytes"] == int((2 * 200 + 30) * row + V * r * 2)  # target and U rows, bonus rows, W2 once
    # no residual draw: W2 is not read
    out0 = b._logit_passes(phases, {"rows": 10.0, "residual": 0.0, "bonus": 5.0}, 256, V, r)
    assert out0["verify_draw"]["bytes"] == int(5 * row)
    # position passes only: no walk entry
    assert "verify_walk" not in b._logit_passes({"verify_draw": {"avg_us": 1.0}}, outcome, 256, V, r)


def test_outcome_counts_leave_sampled_bonus_rows_to_the_draw():
    torch = pytest.importorskip("torch")
    b = _bench()
    ell = torch.tensor([5, 5, 3, 0, 0, 2], dtype=torch.int32)
    temperature = torch.tensor([1.0, 0.0, 0.7, 1.0, 0.0, 1.0])
    add, mean = b._outcome_counter(torch, temperature, ell)
    n = torch.tensor([5, 5, 1, 0, 0, 2], dtype=torch.int32)
    add(n)
    add(torch.tensor([2, 5, 3, 0, 0, 0], dtype=torch.int32))
    m = mean()
    # round 1: rows 6 + 6 + 2 + 1 + 1 + 3 = 19, less the sampled bonus rows of
    # requests 0, 3 and 5 (greedy request 1 and 4 read theirs): 16; residual:
    # request 2; bonus: requests 0, 3, 5
    # round 2: rows 3 + 6 + 4 + 1 + 1 + 1 = 16, less requests 2 and 3: 14;
    # residual: requests 0 and 5; bonus: requests 2 and 3
    assert m == {"rows": (16 + 14) / 2, "residual": (1 + 2) / 2, "bonus": (3 + 2) / 2}
    assert np.isfinite(list(m.values())).all()
