"""Pins for the oracle's confidence-scheduled prefix scheduler.

Checked against the prefix-survival example of the interactive page
(section 04), against full enumeration of every length vector on tiny
inputs, and against closed-form special cases of the cost curve.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
from synth_inputs import CONFIGS, sps_table_toy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, *vals = line.split()
                out[key] = [float(t) for t in vals]
    return out


def _theta(c, ell, sps):
    """Expected-throughput estimate of a length vector, straight from the
    definitions B = sum(1 + ell), tau = sum(1 + sum_{j<=ell} a_j), Theta = tau * SPS(B)."""
    R, gamma = c.shape
    B = int(sum(1 + e for e in ell))
    tau = 0.0
    for r in range(R):
        a = 1.0
        tau += 1.0
        for j in range(ell[r]):
            a *= c[r, j]
            tau += a
    s = sps[B] if B < len(sps) else 0.0
    return tau * s, tau, B


def test_prefix_survival_example_section04():
    g = _golden("prefix_survival_toy.txt")
    c = np.array([g["c"]])
    # a constant SPS makes every extension an improvement, so all three are taken
    ell, theta, tau, B = oracle.schedule(c, np.ones(16))
    assert ell.tolist() == [3]
    assert B == 4
    assert tau == pytest.approx(g["expected_new_tokens"][0], abs=1e-12)
    a = np.cumprod(c[0])
    np.testing.assert_allclose(a, g["a"], atol=1e-12)
    assert theta == pytest.approx(tau)


def test_constant_sps_takes_every_positive_candidate():
    rng = np.random.default_rng(2)
    c = rng.uniform(0.05, 0.95, size=(7, 5))
    c[3, 2] = 0.0  # a_{3,j} = 0 for j >= 2: those candidates are dropped
    ell, theta, tau, B = oracle.schedule(c, np.full(64, 2.0))
    want = [5] * 7
    want[3] = 2
    assert ell.tolist() == want


def test_toy_cost_curve_large_batch_verifies_nothing():
    """With the page's three-request teaching curve, at R >= 32 the marginal
    cost of one more position exceeds the best possible gain, so the first
    candidate already fails to improve Theta: ell = 0 everywhere."""
    cfg = CONFIGS["sched"]
    c = np.random.default_rng((cfg.seed, 5)).beta(8.0, 2.0, size=(cfg.B, cfg.gamma))
    for rho in (0.2, 0.8):
        sps = sps_table_toy(rho, cfg.B * (1 + cfg.gamma) + 1)
        ell, theta, tau, B = oracle.schedule(c, sps)
        assert np.all(ell == 0)
        assert B == cfg.B and tau == cfg.B
        assert theta == pytest.approx(cfg.B * sps[cfg.B], rel=1e-15)
    for R in (32, 64, 200):
        c = np.random.default_rng(R).beta(8.0, 2.0, size=(R, 5))
        ell, *_ = oracle.schedule(c, sps_table_toy(0.2, R * 6 + 1))
        assert np.all(ell == 0)


def test_toy_cost_curve_three_requests_spreads_lengths():
    """Three requests, as in the interactive page: a light load verifies more
    positions than a heavy load."""
    c = np.array([[0.95, 0.9, 0.85, 0.8, 0.7],
                  [0.8, 0.6, 0.5, 0.4, 0.3],
                  [0.6, 0.3, 0.2, 0.1, 0.05]])
    light, *_ = oracle.schedule(c, sps_table_toy(0.0, 19))
    heavy, *_ = oracle.schedule(c, sps_table_toy(1.0, 19))
    assert light.sum() > heavy.sum()
    assert np.all(light >= heavy)


def test_short_sps_table_stops_at_its_end():
    c = np.full((2, 4), 0.9)
    # SPS defined for B = 0..4 only: B = 5 reads SPS = 0, which cannot improve
    ell, theta, tau, B = oracle.schedule(c, np.ones(5))
    assert B == 4 and ell.sum() == 2
    with pytest.raises(ValueError):
        oracle.schedule(c, np.ones(2))  # SPS(R) itself is missing


def test_ties_keep_prefix_order():
    """Equal survival values inside one request (c = 1) must still extend it
    position by position."""
    c = np.array([[1.0, 1.0, 0.5], [0.9, 1.0, 1.0]])
    ell, theta, tau, B = oracle.schedule(c, np.ones(16))
    assert ell.tolist() == [3, 3]
    assert tau == pytest.approx(2 + (1 + 1 + 0.5) + (0.9 + 0.9 + 0.9))


@pytest.mark.parametrize("R,gamma", [(1, 4), (2, 3), (3, 3), (4, 4), (4, 2)])
def test_brute_force_enumeration(R, gamma):
    """Full enumeration of ell in {0..gamma}^R on random confidences and
    random concave-ish cost curves:
      (i)   the greedy lengths maximise tau among all vectors with the same B;
      (ii)  the greedy Theta equals the Theta of the greedy lengths recomputed
            from the definitions, and no single-step extension along the
            descending-a order improves on it;
      (iii) greedy Theta never exceeds the global maximum (it may be below:
            the early stop is what keeps verification lossless)."""
    rng = np.random.default_rng(1000 + 10 * R + gamma)
    below = 0
    for trial in range(40):
        c = rng.uniform(0.0, 1.0, size=(R, gamma))
        n = R * (1 + gamma) + 1
        lin, quad = rng.uniform(0.0, 2.0), rng.uniform(0.0, 0.5)
        sps = 1000.0 / (rng.uniform(5, 30) + lin * np.arange(n) + quad * np.arange(n) ** 2)
        ell, theta, tau, B = oracle.schedule(c, sps)
        th2, tau2, B2 = _theta(c, ell, sps)
        assert B2 == B
        assert tau == pytest.approx(tau2, rel=1e-12)
        assert theta == pytest.approx(th2, rel=1e-12)
        best_tau_same_B = -1.0
        global_best = -1.0
        for vec in itertools.product(range(gamma + 1), repeat=R):
            th, ta, bb = _theta(c, vec, sps)
            global_best = max(global_best, th)
            if bb == B:
                best_tau_same_B = max(best_tau_same_B, ta)
        assert tau >= best_tau_same_B - 1e-12
        assert theta <= global_best + 1e-12
        if theta < global_best - 1e-12:
            below += 1
        # one more step of the greedy order never improves (the early stop)
        a = np.cumprod(c, axis=1)
        nxt = [(a[r, ell[r]], r) for r in range(R) if ell[r] < gamma and a[r, ell[r]] > 0]
        if nxt:
            a_best, r_best = max(nxt, key=lambda t: (t[0], -t[1]))
            ext = list(ell)
            ext[r_best] += 1
            th_ext, _, _ = _theta(c, ext, sps)
            assert th_ext <= theta * (1 + 1e-12)
    # the reported rate is informational; greedy is usually but not always optimal
    assert below <= 40
