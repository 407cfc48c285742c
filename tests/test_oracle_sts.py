"""Pins for the oracle's sequential temperature scaling (page
"DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io), section 4.2: the
confidences are calibrated left to right, each position by a 1-D grid search
for the temperature that minimises the calibration error of the prefix
survival product, earlier positions held fixed; the map keeps the drafts'
order).

The tests fix the result by a hand-worked ECE, by recovering a miscalibration
planted in synthetic outcomes (temperature scaling undoes a known logit
scale), and by the structure the section states: left to right, earlier
positions fixed, samples that did not verify a position do not count there.
"""
import numpy as np
import pytest

import oracle


def test_ece_hand_example():
    """Two bins [0, 1/2) and [1/2, 1], tau = 1 (c unchanged):
    bin 0 holds c = 0.2, 0.4 with outcomes 0, 1: |1 - 0.6| = 0.4;
    bin 1 holds c = 0.7, 0.9 with outcomes 1, 0: |1 - 1.6| = 0.6;
    ECE = (0.4 + 0.6) / 4 = 0.25."""
    c = np.array([[0.2], [0.4], [0.7], [0.9]], np.float32)
    n = np.array([0, 1, 1, 0], np.int32)
    tau, ece, eg = oracle.sts_fit(c, n, np.array([1.0], np.float32), n_bins=2)
    assert tau[0] == 1.0
    assert ece[0] == pytest.approx(0.25, abs=1e-7)  # the float32 inputs
    # two samples in the same bin with outcome 1: the gap is 2 - (c1 + c2)
    tau, ece, _ = oracle.sts_fit(np.array([[0.55], [0.65]], np.float32), np.array([1, 1], np.int32),
                                 np.array([1.0], np.float32), n_bins=2)
    assert ece[0] == pytest.approx((2.0 - 1.2) / 2, abs=1e-7)


def _planted(N, scales, seed):
    """Outcomes from true conditional logits s_k ~ N(0.8, 1.5): position k
    survives iff position k - 1 did and a Bernoulli(sigmoid(s_k)) draw says
    so.  The reported confidences are sigmoid(scale_k * s_k): scale 2 is
    overconfident, 0.5 underconfident.  Temperature scaling undoes it at
    tau_k = scale_k."""
    rng = np.random.default_rng(seed)
    gamma = len(scales)
    s = rng.normal(0.8, 1.5, (N, gamma))
    accept = rng.uniform(size=(N, gamma)) < 1.0 / (1.0 + np.exp(-s))
    n = np.argmin(np.concatenate([accept, np.zeros((N, 1), bool)], axis=1), axis=1).astype(np.int32)
    c = (1.0 / (1.0 + np.exp(-np.asarray(scales) * s))).astype(np.float32)
    return c, n


def test_recovers_planted_temperatures_left_to_right():
    c, n = _planted(200_000, [2.0, 0.5, 1.0], seed=1)
    grid = np.round(np.arange(0.25, 4.0001, 0.05), 2).astype(np.float32)
    tau, ece, eg = oracle.sts_fit(c, n, grid)
    np.testing.assert_allclose(tau, [2.0, 0.5, 1.0], atol=0.15)
    # calibration brings the error down to sampling noise
    assert np.all(ece < 0.01)
    raw = eg[:, np.argmin(np.abs(grid - 1.0))]  # tau = 1, no scaling
    assert raw[0] > 3 * ece[0] and raw[1] > 3 * ece[1]


def test_earlier_positions_are_held_fixed():
    """tau_1 does not look at position 2; tau_2 is fitted on top of the
    calibrated position 1, so changing position 1's confidences moves it."""
    c, n = _planted(50_000, [2.0, 0.5], seed=2)
    grid = np.round(np.arange(0.25, 4.0001, 0.05), 2).astype(np.float32)
    tau, _, _ = oracle.sts_fit(c, n, grid)
    c2 = c.copy()
    c2[:, 1] = np.float32(0.5)
    tau2, _, _ = oracle.sts_fit(c2, n, grid)
    assert tau2[0] == tau[0]
    c3 = c.copy()
    c3[:, 0] = np.float32(0.999)
    tau3, _, _ = oracle.sts_fit(c3, n, grid)
    assert tau3[1] != tau[1]


def test_unverified_samples_do_not_count():
    """Samples with ell < k have no outcome at k: adding them changes nothing
    there; a position nobody verified keeps tau = 1 with ECE NaN."""
    c, n = _planted(20_000, [2.0, 1.0, 0.5], seed=3)
    grid = np.round(np.arange(0.25, 4.0001, 0.05), 2).astype(np.float32)
    tau, ece, _ = oracle.sts_fit(c, n, grid)
    rng = np.random.default_rng(9)
    extra_c = rng.uniform(0.01, 0.99, (5000, 3)).astype(np.float32)
    extra_n = rng.integers(0, 4, 5000).astype(np.int32)
    cc = np.concatenate([c, extra_c])
    nn = np.concatenate([n, extra_n])
    ell = np.concatenate([np.full(len(c), 3), np.zeros(5000)]).astype(np.int32)
    tau2, ece2, _ = oracle.sts_fit(cc, nn, grid, ell=ell)
    np.testing.assert_array_equal(tau2, tau)
    np.testing.assert_allclose(ece2, ece, rtol=1e-12)
    tau3, ece3, _ = oracle.sts_fit(c, n, grid, ell=np.full(len(c), 1, np.int32))
    assert tau3[0] == tau[0] and np.all(tau3[1:] == 1.0) and np.all(np.isnan(ece3[1:]))


def test_grid_ties_and_non_positive_temperatures():
    c, n = _planted(5000, [1.5], seed=4)
    tau, _, eg = oracle.sts_fit(c, n, np.array([-1.0, 0.0, 1.5, 1.5, 3.0], np.float32))
    assert tau[0] == 1.5
    assert np.all(np.isinf(eg[0, :2])) and eg[0, 2] == eg[0, 3]


def test_scaling_keeps_the_order():
    """sigmoid(logit(c) / tau) is increasing in c for tau > 0: the calibrated
    confidences rank the drafts as the raw ones do."""
    rng = np.random.default_rng(5)
    c = np.sort(rng.uniform(0.001, 0.999, 1000))
    for tau in (0.3, 1.0, 2.7):
        cp = 1.0 / (1.0 + np.exp(-(np.log(c) - np.log1p(-c)) / tau))
        assert np.all(np.diff(cp) > 0)


def test_temperature_of_the_head_is_the_scaling_of_its_confidence():
    """The head evaluated with temperatures tau_k (the calibrated head) gives
    sigmoid(logit(c_k) / tau_k) of the raw head's c_k; tau = 1 changes nothing."""
    rng = np.random.default_rng(7)
    B, gamma, d, V, r = 6, 4, 8, 20, 4
    h = rng.standard_normal((B, gamma, d)).astype(np.float32)
    w = (rng.standard_normal(d + r) * 0.5).astype(np.float32)
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    c, _ = oracle.confidence(h, w, W1, anchor, x)
    tau = np.array([0.5, 1.0, 2.0, 3.5], np.float32)
    ct, at = oracle.confidence(h, w, W1, anchor, x, tau=tau)
    want = 1.0 / (1.0 + np.exp(-(np.log(c) - np.log1p(-c)) / tau))
    np.testing.assert_allclose(ct, want, rtol=1e-12)
    np.testing.assert_allclose(at, np.cumprod(want, axis=1), rtol=1e-12)
    c1, _ = oracle.confidence(h, w, W1, anchor, x, tau=np.ones(gamma, np.float32))
    np.testing.assert_array_equal(c1, c)
