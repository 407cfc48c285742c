"""Pins for the oracle's production-style scheduler ("DeepSeek DSpark
explained" (share.concentrate1.com), section 04, the paragraph on the strict
implementation: capacity from the previous two steps' predictions, then a
sort of the current candidates, no early stop on the current step).

The fixed-capacity scheduler is checked against the page's survival example,
against the synchronous scheduler (equal when the capacity is the one the
synchronous rule would pick), and against brute force: with survival
products non-increasing along each request, taking candidates in descending
order under the prefix rule maximises the expected emitted tokens tau for
the capacity.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from synth_inputs import sps_table_toy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_survival_example_section04_by_capacity():
    """One request with c = 0.8, 0.8, 0.8: capacity 4 (the anchor plus three
    drafts) expects 1 + 0.8 + 0.64 + 0.512 = 2.952 tokens, capacity 2 expects
    1.8; capacity 1 verifies only the anchor position."""
    vals = {}
    with open(os.path.join(GOLDEN, "prefix_survival_toy.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, *v = line.split()
                vals[k] = [float(t) for t in v]
    c = np.array([vals["c"]])
    ell, tau, B = oracle.schedule_capacity(c, 4)
    assert ell.tolist() == [3] and B == 4 and tau == pytest.approx(vals["expected_new_tokens"][0], abs=1e-12)
    ell, tau, B = oracle.schedule_capacity(c, 2)
    assert ell.tolist() == [1] and tau == pytest.approx(1.8, abs=1e-12)
    ell, tau, B = oracle.schedule_capacity(c, 1)
    assert ell.tolist() == [0] and B == 1 and tau == 1.0


@pytest.mark.parametrize("seed", range(12))
def test_capacity_of_the_synchronous_choice_gives_its_lengths(seed):
    rng = np.random.default_rng(seed)
    R, gamma = int(rng.integers(1, 30)), int(rng.integers(1, 7))
    c = rng.beta(6.0, 2.0, size=(R, gamma))
    for rho in (0.0, 0.3, 1.0):
        sps = sps_table_toy(rho, R * (1 + gamma) + 1) if rho > 0 else np.full(R * (1 + gamma) + 1, 1.0)
        ell_s, theta, tau_s, B_s = oracle.schedule(c, sps)
        ell, tau, B = oracle.schedule_capacity(c, B_s)
        assert ell.tolist() == ell_s.tolist() and B == B_s and tau == tau_s


@pytest.mark.parametrize("R,gamma", [(1, 3), (2, 2), (2, 3), (3, 2), (3, 3)])
def test_brute_force_best_tau_for_each_capacity(R, gamma):
    rng = np.random.default_rng(R * 10 + gamma)
    for trial in range(6):
        c = rng.uniform(0.05, 1.0, size=(R, gamma))
        a = np.cumprod(c, axis=1)
        best = {}
        for ell in itertools.product(range(gamma + 1), repeat=R):
            B = R + sum(ell)
            t = R + sum(a[r, :ell[r]].sum() for r in range(R))
            best[B] = max(best.get(B, -1.0), t)
        for cap in range(R, R * (1 + gamma) + 1):
            ell, tau, B = oracle.schedule_capacity(c, cap)
            assert B == cap
            assert tau == pytest.approx(best[cap], rel=1e-12)


def test_capacity_bounds_and_monotonicity():
    rng = np.random.default_rng(3)
    R, gamma = 12, 5
    c = rng.uniform(0.01, 1.0, size=(R, gamma))
    ell, tau, B = oracle.schedule_capacity(c, 0)
    assert np.all(ell == 0) and B == R and tau == R
    ell, tau, B = oracle.schedule_capacity(c, 10 * R * gamma)
    assert np.all(ell == gamma) and B == R * (1 + gamma)
    prev = np.zeros(R, np.int32)
    for cap in range(R, R * (1 + gamma) + 1):
        ell, _, B = oracle.schedule_capacity(c, cap)
        assert B == cap and np.all(ell >= prev) and (ell - prev).sum() == (1 if cap > R else 0)
        prev = ell
    # zero-survival candidates are never taken
    c[0, 2] = 0.0
    ell, _, B = oracle.schedule_capacity(c, 10 * R * gamma)
    assert ell[0] == 2 and B == R * (1 + gamma) - (gamma - 2)


def test_history_capacity():
    # B / R of the two previous steps: 3.0 and 2.0, mean 2.5, for 10 requests: 25
    assert oracle.history_capacity([30, 20], [10, 10], 10, 5) == 25
    # per-request rates carry over to a batch of another size: 2 and 3 a request, 7 requests -> 17.5 -> 18
    assert oracle.history_capacity([30, 30], [15, 10], 7, 5) == 18
    # a step without requests is skipped; no usable history: verify everything
    assert oracle.history_capacity([30, 0], [10, 0], 4, 5) == 12
    assert oracle.history_capacity([0, 0], [0, 0], 4, 5) == 24
    # clamped to [R, R (1 + gamma)]
    assert oracle.history_capacity([70, 70], [10, 10], 10, 5) == 60
    assert oracle.history_capacity([1, 1], [10, 10], 10, 5) == 10
