"""The library's host scheduler (heap merge) against the oracle's
sort-based scheduler: bit-identical lengths, Theta, tau and B."""
import numpy as np
import pytest

import draft_sampling_verification_02_amd as ds
import oracle
from synth_inputs import CONFIGS, sps_table_toy


def _same(c, sps):
    got = ds.dspark_schedule(c, sps)
    want = oracle.schedule(c, sps)
    assert got[0].tolist() == want[0].tolist()
    assert got[1] == want[1] and got[2] == want[2] and got[3] == want[3]
    return got


def test_scheduled_config_literal_and_grouped():
    cfg = CONFIGS["sched"]
    c = np.random.default_rng((cfg.seed, 5)).beta(8.0, 2.0, size=(cfg.B, cfg.gamma))
    for rho in (0.2, 0.8):
        sps = sps_table_toy(rho, cfg.B * (1 + cfg.gamma) + 1)
        ell, *_ = _same(c, sps)
        assert np.all(ell == 0)
        # 256 independent groups of 4 requests: real spread of lengths
        grouped = []
        for g in range(cfg.B // 4):
            e, *_ = _same(c[4 * g:4 * g + 4], sps_table_toy(rho, 4 * (1 + cfg.gamma) + 1))
            grouped.append(e)
        grouped = np.concatenate(grouped)
        assert grouped.min() >= 0 and grouped.max() <= cfg.gamma
        assert len(np.unique(grouped)) >= 3


@pytest.mark.parametrize("seed", range(30))
def test_random_inputs_match_oracle(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(0, 40))
    gamma = int(rng.integers(1, 9))
    c = rng.uniform(0, 1, size=(R, gamma))
    if seed % 3 == 0:
        c[rng.uniform(size=c.shape) < 0.2] = 1.0  # ties inside requests
    if seed % 4 == 1:
        c[rng.uniform(size=c.shape) < 0.1] = 0.0  # zero survival
    if seed % 5 == 2:
        c = np.round(c, 1)  # ties across requests
    n = R * (1 + gamma) + 1
    kind = seed % 3
    if kind == 0:
        sps = 1000.0 / (10 + rng.uniform(0, 2) * np.arange(n) + rng.uniform(0, 0.3) * np.arange(n) ** 2)
    elif kind == 1:
        sps = np.full(n, 3.0)
    else:
        sps = 1000.0 / (10 + np.arange(n)) [: max(R + 1, n // 2)]
    _same(c, sps)


def test_large_batch_matches_oracle():
    rng = np.random.default_rng(7)
    c = rng.beta(8, 2, size=(4096, 8))
    for lin in (0.001, 0.01, 0.1):
        n = 4096 * 9 + 1
        sps = 1000.0 / (50 + lin * np.arange(n))
        _same(c, sps)


@pytest.mark.parametrize("seed", range(20))
def test_capacity_scheduler_matches_oracle(seed):
    """The library's heap merge with a fixed capacity against the oracle's
    sort: identical lengths, tau and B for every capacity."""
    rng = np.random.default_rng(100 + seed)
    R = int(rng.integers(0, 50))
    gamma = int(rng.integers(1, 9))
    c = rng.beta(6.0, 2.0, size=(R, gamma))
    c[rng.uniform(size=c.shape) < 0.05] = 0.0
    c[:, 0][rng.uniform(size=R) < 0.1] = 1.0
    for cap in sorted({0, R, R + 1, R + R * gamma // 3, R * (1 + gamma), R * (1 + gamma) + 5,
                       int(rng.integers(0, R * (1 + gamma) + 1))}):
        got = ds.dspark_schedule_capacity(c, cap)
        want = oracle.schedule_capacity(c, cap)
        assert got[0].tolist() == want[0].tolist() and got[1] == want[1] and got[2] == want[2]


def test_history_capacity_matches_oracle():
    rng = np.random.default_rng(7)
    for _ in range(200):
        gamma = int(rng.integers(1, 9))
        R = int(rng.integers(0, 300))
        Rh = rng.integers(0, 300, 2).astype(np.int32)
        Bh = (Rh * rng.uniform(1.0, 1.0 + gamma, 2)).astype(np.int32)
        n = int(rng.integers(0, 3))
        assert ds.dspark_history_capacity(Bh[:n], Rh[:n], R, gamma) == oracle.history_capacity(Bh[:n], Rh[:n], R, gamma)


def test_capacity_scheduler_rejects_bad_confidences():
    with pytest.raises(ds.DSparkError):
        ds.dspark_schedule_capacity(np.array([[0.5, 1.5]]), 3)
    with pytest.raises(ds.DSparkError):
        ds.dspark_schedule_capacity(np.array([[np.nan]]), 3)
