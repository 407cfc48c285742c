"""Pins for the oracle's confidence head, prefix survival and per-position
acceptance probability.

Confidence head (page "DSpark：DeepSeek 线上跑的投机解码..." (marsggbo.github.io),
section 4.1): c_k = sigmoid(w . [h_k, W1[x_{k-1}]]), no bias; prefix
survival a_k = c_1 ... c_k (same page, section 4.2; "DeepSeek DSpark
explained" (share.concentrate1.com), section 04).  Acceptance probability
(section 4.1 of the first page; section 05 of the second): alpha_k =
sum_v min(p_k, q_k) = 1 - TV(p_k, q_k).

Each test checks the oracle against something fixed outside it: the pages'
worked examples (tests/golden/), values worked out by hand, closed forms of
the sigmoid, and the rejection rule itself (Monte-Carlo acceptance
frequencies of the oracle's verify, which shares no summation with the
alpha computation).
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


# ---------------------------------------------------------------- confidence head

def test_prefix_survival_toy_section04():
    """c_1 = c_2 = c_3 = 0.8 gives a_3 = 0.512 and 1 + a_1 + a_2 + a_3 expected
    new tokens.  The head's logit is made ln 4 (sigmoid(ln 4) = 4/5) by a
    one-dimensional h = 1 and w_h = ln 4, with the W1 half of w zero."""
    g = _golden("prefix_survival_toy.txt")
    c_exp = [float(t) for t in g["c"]]
    a_exp = [float(t) for t in g["a"]]
    gamma = len(c_exp)
    V, r = 5, 4
    rng = np.random.default_rng(3)
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    h = np.ones((1, gamma, 1), np.float32)
    w = np.zeros(1 + r, np.float32)
    w[0] = np.float32(math.log(4.0))
    c, a = oracle.confidence(h, w, W1, np.array([1], np.int32), np.array([[2, 0, 4]], np.int32))
    # ln 4 is rounded to float32, so sigmoid moves by at most its slope 0.16 x 2^-24 x ln 4
    np.testing.assert_allclose(c[0], c_exp, atol=1e-7)
    np.testing.assert_allclose(a[0], a_exp, atol=1e-7)
    assert 1.0 + a[0].sum() == pytest.approx(float(g["expected_new_tokens"][0]), abs=1e-6)


def test_confidence_hand_example():
    """d = 2, r = 2, anchor 2, drafts (0, 1, 2).  The logits, worked out by hand
    with w = (0.5, -0.25 | 1, 3):
      k = 1: h = (1, 2),  W1[x_0 = 2] = (2, -1): 0.5 - 0.5 + 2 - 3 = -1
      k = 2: h = (0, 4),  W1[x_1 = 0] = (1, 0):  0 - 1 + 1 + 0     =  0
      k = 3: h = (-2, 0), W1[x_2 = 1] = (0, 1):  -1 + 0 + 0 + 3    =  2
    sigmoid(-1) = 0.2689414213699951, sigmoid(0) = 0.5,
    sigmoid(2) = 0.8807970779778823.  Swapping the two halves of w, or
    gathering W1[x_k] instead of W1[x_{k-1}], changes every one of them."""
    W1 = np.array([[1, 0], [0, 1], [2, -1]], np.float32)
    w = np.array([0.5, -0.25, 1.0, 3.0], np.float32)
    h = np.array([[[1, 2], [0, 4], [-2, 0]]], np.float32)
    c, a = oracle.confidence(h, w, W1, np.array([2], np.int32), np.array([[0, 1, 2]], np.int32))
    c_exp = np.array([0.2689414213699951, 0.5, 0.8807970779778823])
    np.testing.assert_allclose(c[0], c_exp, rtol=0, atol=1e-15)
    np.testing.assert_allclose(a[0], [c_exp[0], c_exp[0] * 0.5, c_exp[0] * 0.5 * c_exp[2]], rtol=1e-15)


def test_confidence_zero_weight_is_one_half():
    rng = np.random.default_rng(5)
    B, gamma, d, V, r = 3, 6, 7, 11, 4
    h = rng.standard_normal((B, gamma, d)).astype(np.float32)
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    c, a = oracle.confidence(h, np.zeros(d + r, np.float32), W1, np.zeros(B, np.int32), x)
    assert np.all(c == 0.5)
    np.testing.assert_allclose(a, np.broadcast_to(0.5 ** np.arange(1, gamma + 1), (B, gamma)), rtol=1e-15)


def test_confidence_sign_flip_complements():
    """sigmoid(-s) = 1 - sigmoid(s): negating w turns every c_k into 1 - c_k;
    survival is a product of factors in (0, 1), so it never increases."""
    rng = np.random.default_rng(6)
    B, gamma, d, V, r = 4, 5, 16, 20, 8
    h = rng.standard_normal((B, gamma, d)).astype(np.float32)
    w = (rng.standard_normal(d + r) * 0.4).astype(np.float32)
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    c, a = oracle.confidence(h, w, W1, anchor, x)
    cn, _ = oracle.confidence(h, -w, W1, anchor, x)
    np.testing.assert_allclose(cn, 1.0 - c, atol=1e-15)
    assert np.all((c > 0) & (c < 1))
    assert np.all(np.diff(a, axis=1) <= 0)
    np.testing.assert_allclose(a[:, 0], c[:, 0], rtol=0)


def test_confidence_depends_on_the_prefix_only():
    """c_k reads h_k and x_{k-1}: changing x_k leaves c_1..c_k as they were."""
    rng = np.random.default_rng(8)
    B, gamma, d, V, r = 2, 4, 3, 9, 4
    h = rng.standard_normal((B, gamma, d)).astype(np.float32)
    w = rng.standard_normal(d + r).astype(np.float32)
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    anchor = np.array([1, 7], np.int32)
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    c, _ = oracle.confidence(h, w, W1, anchor, x)
    x2 = x.copy()
    x2[:, 2] = (x2[:, 2] + 1) % V
    c2, _ = oracle.confidence(h, w, W1, anchor, x2)
    np.testing.assert_array_equal(c[:, :3], c2[:, :3])
    assert np.all(c[:, 3] != c2[:, 3])


# ---------------------------------------------------------------- acceptance probability

def _toy_inputs(q, p, gamma, B=1):
    V = len(q)
    W = np.zeros((V, 1), np.float32)
    U = np.ascontiguousarray(np.broadcast_to(np.log(q).astype(np.float32), (B, gamma, V)))
    return U, W, V


def test_acceptance_toy_section05():
    """q = (0.70, 0.18, 0.12), p = (0.50, 0.30, 0.20): accepted mass
    (0.50, 0.18, 0.12), acceptance probability 0.80, at every verified
    position; NaN past ell."""
    g = _golden("exact_sampling_toy.txt")
    q = [float(t) for t in g["q"]]
    p = [float(t) for t in g["p"]]
    gamma = 3
    U, W, V = _toy_inputs(q, p, gamma, B=2)
    ell = np.array([3, 1], np.int32)
    nrows = int((1 + ell).sum())
    target = np.ascontiguousarray(np.broadcast_to(np.log(p).astype(np.float32), (nrows, V)))
    x = np.zeros((2, gamma), np.int32)
    alpha = oracle.acceptance(target, ell, U, W, W, np.zeros(2, np.int32), x, np.ones(2, np.float32))
    expected = float(g["acceptance"][0])
    # float32 logits move each probability by ~1e-7 relative
    np.testing.assert_allclose(alpha[0], expected, atol=1e-6)
    assert alpha[1, 0] == pytest.approx(expected, abs=1e-6)
    assert np.all(np.isnan(alpha[1, 1:]))


def test_acceptance_identical_distributions_is_one():
    rng = np.random.default_rng(9)
    B, gamma, V = 3, 4, 50
    U = rng.normal(0, 3, (B, gamma, V)).astype(np.float32)
    W = np.zeros((V, 2), np.float32)
    ell = np.full(B, gamma, np.int32)
    target = np.zeros((int((1 + ell).sum()), V), np.float32)
    for b in range(B):
        target[b * (gamma + 1): b * (gamma + 1) + gamma] = U[b]
    T = np.array([1.0, 0.5, 2.0], np.float32)
    alpha = oracle.acceptance(target, ell, U, W, W, np.zeros(B, np.int32), np.zeros((B, gamma), np.int32), T)
    np.testing.assert_allclose(alpha, 1.0, atol=1e-12)


def test_acceptance_disjoint_supports_is_zero():
    neg = -np.inf
    U = np.array([[[0.0, 1.0, neg, neg]]], np.float32)
    target = np.array([[neg, neg, 0.0, 2.0], [0, 0, 0, 0]], np.float32)
    W = np.zeros((4, 1), np.float32)
    alpha = oracle.acceptance(target, np.array([1], np.int32), U, W, W, np.zeros(1, np.int32),
                              np.zeros((1, 1), np.int32), np.ones(1, np.float32))
    assert alpha[0, 0] == 0.0


def _markov_case(B, gamma, V, r, T, seed):
    """Identical requests with a real Markov bias: U, t rows shared, W1/W2
    random; each request draws its own Philox streams."""
    rng = np.random.default_rng(seed)
    Urows = rng.normal(0, 1.0, (gamma, V)).astype(np.float32)
    U = np.ascontiguousarray(np.broadcast_to(Urows, (B, gamma, V)))
    W1 = rng.normal(0, 0.6, (V, r)).astype(np.float32)
    W2 = rng.normal(0, 0.6, (V, r)).astype(np.float32)
    trows = (Urows + rng.normal(0, 1.0, (gamma, V))).astype(np.float32)
    ell = np.full(B, gamma, np.int32)
    target = np.zeros((B * (gamma + 1), V), np.float32)
    target.reshape(B, gamma + 1, V)[:, :gamma] = trows
    target.reshape(B, gamma + 1, V)[:, gamma] = trows[-1]
    anchor = np.full(B, 3, np.int32)
    temp = np.full(B, T, np.float32)
    return U, W1, W2, target, ell, anchor, temp


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_acceptance_is_the_rejection_rule_pass_rate(T):
    """alpha_1 is the probability that the first draft passes; alpha_2 is the
    pass rate at position 2 of the requests whose first draft passed, given
    their x_1 (the target rows here do not depend on the prefix)."""
    B, gamma, V, r = 60_000, 2, 24, 4
    U, W1, W2, target, ell, anchor, temp = _markov_case(B, gamma, V, r, T, seed=11)
    d = oracle.draft(U, W1, W2, anchor, temp, seed=5, round_id=2)
    v = oracle.verify(target, ell, U, W1, W2, anchor, d["x"], temp, seed=5, round_id=2)
    alpha = oracle.acceptance(target, ell, U, W1, W2, anchor, d["x"], temp)
    a1 = alpha[0, 0]
    assert np.all(alpha[:, 0] == a1)  # the same for every request: x_0 is shared
    rate1 = (v["n"] >= 1).mean()
    assert abs(rate1 - a1) < 4.5 * math.sqrt(a1 * (1 - a1) / B)
    passed = v["n"] >= 1
    rate2 = (v["n"][passed] >= 2).mean()
    mean_a2 = alpha[passed, 1].mean()
    nb = passed.sum()
    assert abs(rate2 - mean_a2) < 4.5 * math.sqrt(mean_a2 * (1 - mean_a2) / nb)
    # alpha_2 really depends on x_1 through the Markov bias
    assert alpha[passed, 1].std() > 1e-3


def test_acceptance_complements_the_residual_mass():
    """At a sampled rejection at j the residual mass S = sum max(p_j - q_j, 0)
    is TV(p_j, q_j), so alpha_j = 1 - S."""
    B, gamma, V, r = 400, 3, 40, 4
    U, W1, W2, target, ell, anchor, temp = _markov_case(B, gamma, V, r, 1.0, seed=12)
    d = oracle.draft(U, W1, W2, anchor, temp, seed=8, round_id=0)
    v = oracle.verify(target, ell, U, W1, W2, anchor, d["x"], temp, seed=8, round_id=0)
    alpha = oracle.acceptance(target, ell, U, W1, W2, anchor, d["x"], temp)
    rej = np.nonzero(v["n"] < gamma)[0]
    assert len(rej) > 50
    j = v["n"][rej]  # 0-based position of the rejection
    np.testing.assert_allclose(alpha[rej, j], 1.0 - v["resid"][rej], atol=1e-12)


def test_acceptance_greedy_is_the_match_indicator():
    """T = 0: alpha_k = 1 exactly where the greedy rule accepts x_k (x_k equal
    to the lowest-index argmax of t_k), also past the first rejection."""
    rng = np.random.default_rng(13)
    B, gamma, V, r = 64, 4, 6, 2
    U = rng.normal(0, 1, (B, gamma, V)).astype(np.float32)
    W1 = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    W2 = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    ell = np.full(B, gamma, np.int32)
    target = np.round(rng.normal(0, 1, (B * (gamma + 1), V)), 0).astype(np.float32)  # ties included
    anchor = rng.integers(0, V, B).astype(np.int32)
    temp = np.zeros(B, np.float32)
    d = oracle.draft(U, W1, W2, anchor, temp, seed=0, round_id=0)
    alpha = oracle.acceptance(target, ell, U, W1, W2, anchor, d["x"], temp)
    t = target.reshape(B, gamma + 1, V)[:, :gamma]
    am = np.argmax(t, axis=-1)  # numpy's argmax takes the first maximum
    np.testing.assert_array_equal(alpha, (am == d["x"]).astype(np.float64))
    v = oracle.verify(target, ell, U, W1, W2, anchor, d["x"], temp, seed=0, round_id=0)
    for b in range(B):
        n = v["n"][b]
        assert np.all(alpha[b, :n] == 1.0)
        if n < gamma:
            assert alpha[b, n] == 0.0


def test_acceptance_ragged_rows_and_offsets():
    """Packed and explicitly offset target rows give the same alpha; positions
    past ell are NaN; ell = 0 verifies nothing."""
    rng = np.random.default_rng(14)
    B, gamma, V, r = 5, 3, 30, 4
    U = rng.normal(0, 2, (B, gamma, V)).astype(np.float32)
    W1 = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    W2 = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    ell = np.array([3, 0, 2, 1, 3], np.int32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    temp = np.array([1.0, 1.0, 0.8, 1.5, 1.0], np.float32)
    packed = rng.normal(0, 2, (int((1 + ell).sum()), V)).astype(np.float32)
    alpha = oracle.acceptance(packed, ell, U, W1, W2, anchor, x, temp)
    for b in range(B):
        assert np.all(np.isnan(alpha[b, ell[b]:]))
        assert np.all((alpha[b, :ell[b]] > 0) & (alpha[b, :ell[b]] < 1))
    # the same rows scattered with gaps, addressed through explicit offsets
    off = np.zeros(B, np.int32)
    spread = np.full((int((1 + ell).sum()) + 3 * B, V), np.nan, np.float32)
    acc, pos = 0, 0
    for b in range(B):
        pos += 3
        off[b] = pos
        spread[pos: pos + 1 + ell[b]] = packed[acc: acc + 1 + ell[b]]
        acc += 1 + ell[b]
        pos += 1 + ell[b]
    alpha2 = oracle.acceptance(spread, ell, U, W1, W2, anchor, x, temp, row_offsets=off)
    np.testing.assert_array_equal(np.isnan(alpha), np.isnan(alpha2))
    np.testing.assert_allclose(alpha2[~np.isnan(alpha)], alpha[~np.isnan(alpha)], rtol=0, atol=0)


def test_acceptance_rejects_bad_lengths():
    U = np.zeros((1, 2, 4), np.float32)
    W = np.zeros((4, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.acceptance(np.zeros((4, 4), np.float32), np.array([3], np.int32), U, W, W,
                          np.zeros(1, np.int32), np.zeros((1, 2), np.int32), np.ones(1, np.float32))
