"""Pins for the oracle's draft sampler and exact verification.

Each test checks the oracle against something fixed outside it: the pages'
worked examples (tests/golden/), closed forms of speculative sampling, or
textbook identities (Gumbel-max, inverse-CDF sampling, greedy decoding).
Monte-Carlo checks use independent requests of one batch as samples: each
request index draws its own Philox stream.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEG = -np.inf


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


def _chi2_crit(dof, alpha=1e-3):
    from scipy.stats import chi2
    return chi2.ppf(1 - alpha, dof)


def _chi2(counts, probs):
    counts = np.asarray(counts, float)
    probs = np.asarray(probs, float)
    n = counts.sum()
    exp = n * probs
    keep = exp > 0
    assert np.all(counts[~keep] == 0), "mass on a zero-probability outcome"
    return float(((counts[keep] - exp[keep]) ** 2 / exp[keep]).sum()), int(keep.sum()) - 1


def _broadcast_draft_inputs(Urows, B):
    """U [B, gamma, V] with the same rows for every request."""
    Urows = np.asarray(Urows, np.float32)
    return np.ascontiguousarray(np.broadcast_to(Urows, (B,) + Urows.shape))


# ---------------------------------------------------------------- draft

def test_markov_bias_toy_section03():
    """Two continuations, base scores equal, bias ln 9 on the compatible one:
    q = 0.9 / 0.1 (section 03 toy), exercised through the W1 gather and the
    W2 product.  Tokens: 0, 1 = two first words; 2, 3 = their compatible
    continuations; 4 = the anchor."""
    g = _golden("markov_bias_toy.txt")
    q_hi, q_lo = float(g["q_compatible"][0]), float(g["q_other"][0])
    ln9 = math.log(9.0)
    V, r = 5, 2
    W1 = np.zeros((V, r), np.float32)
    W1[0] = (1, 0)
    W1[1] = (0, 1)
    W2 = np.zeros((V, r), np.float32)
    W2[2] = (ln9, 0)  # continuation of token 0
    W2[3] = (0, ln9)  # continuation of token 1
    U1 = [0, 0, NEG, NEG, NEG]
    U2 = [NEG, NEG, 0, 0, NEG]
    B = 200_000
    U = _broadcast_draft_inputs([U1, U2], B)
    out = oracle.draft(U, W1, W2, np.full(B, 4), np.ones(B, np.float32), seed=11, round_id=0)
    x = out["x"]
    assert set(np.unique(x[:, 0])) <= {0, 1}
    assert set(np.unique(x[:, 1])) <= {2, 3}
    np.testing.assert_allclose(out["qx"][:, 0], 0.5, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out["lse"][:, 0], math.log(2.0), atol=1e-15)
    np.testing.assert_allclose(out["lse"][:, 1], math.log(10.0), atol=1e-14)
    compatible = x[:, 1] == x[:, 0] + 2
    np.testing.assert_allclose(out["qx"][compatible, 1], q_hi, atol=1e-14)
    np.testing.assert_allclose(out["qx"][~compatible, 1], q_lo, atol=1e-14)
    frac = compatible.mean()
    assert abs(frac - q_hi) < 4 * math.sqrt(q_hi * q_lo / B)
    assert abs((x[:, 0] == 0).mean() - 0.5) < 4 * math.sqrt(0.25 / B)


def test_gumbel_max_matches_softmax():
    """Textbook: argmax(z + Gumbel) is distributed as softmax(z)."""
    z = np.array([0.3, -1.0, 2.0, 0.0, 1.2, -0.4], np.float32)
    V = len(z)
    B = 300_000
    U = _broadcast_draft_inputs([z], B)
    W = np.zeros((V, 1), np.float32)
    out = oracle.draft(U, W, W, np.zeros(B), np.ones(B, np.float32), seed=3, round_id=9)
    p = np.exp(z.astype(np.float64) - np.log(np.exp(z.astype(np.float64)).sum()))
    chi2, dof = _chi2(np.bincount(out["x"][:, 0], minlength=V), p)
    assert chi2 < _chi2_crit(dof)
    np.testing.assert_allclose(out["qx"][:, 0], p[out["x"][:, 0]], rtol=1e-13)


def test_two_level_draw_matches_softmax_across_tiles():
    """The draft sampler (a Gumbel race over 32-entry tile logsumexps, then
    over the entries of the winning tile) is an exact draw from softmax(z):
    chi-square over a vocabulary spanning several tiles and a ragged tail,
    with -inf entries that must never come out."""
    rng = np.random.default_rng(12)
    V = 75  # tiles of 32, 32, 11
    z = (rng.standard_normal(V) * 1.2).astype(np.float32)
    z[[3, 40, 74]] = -np.inf
    B = 400_000
    U = _broadcast_draft_inputs([z], B)
    W = np.zeros((V, 1), np.float32)
    out = oracle.draft(U, W, W, np.zeros(B), np.ones(B, np.float32), seed=6, round_id=2)
    zz = z.astype(np.float64)
    p = np.exp(zz - zz[np.isfinite(zz)].max())
    p /= p.sum()
    counts = np.bincount(out["x"][:, 0], minlength=V)
    assert counts[3] == counts[40] == counts[74] == 0
    # merge bins with expected count < 5
    exp_ = B * p
    keep = exp_ >= 5
    c2 = (((counts[keep] - exp_[keep]) ** 2) / exp_[keep]).sum()
    rest_c, rest_e = counts[~keep].sum(), exp_[~keep].sum()
    if rest_e > 0:
        c2 += (rest_c - rest_e) ** 2 / rest_e
    assert c2 < _chi2_crit(int(keep.sum()))


def test_two_level_draw_brute_force():
    """Each sampled draft equals the two-level argmax recomputed here from the
    raw Philox words with numpy: tile t maximising logsumexp(z over t) plus
    tile noise (stream 3, index t), then the entry of t maximising z plus
    entry noise (stream 0, index v); the reported margin is the smaller
    top-two gap of the two levels."""
    rng = np.random.default_rng(21)
    V, B, seed, rid, k = 70, 300, 17, 5, 1
    z = (rng.standard_normal((B, 1, V)) * 2).astype(np.float32)
    W = np.zeros((V, 1), np.float32)
    out = oracle.draft(z, W, W, np.zeros(B), np.ones(B, np.float32), seed=seed, round_id=rid)

    def g(stream, b, i):
        w = np.array([oracle.random_word(seed, rid, stream, k, b, j) for j in i], np.uint64)
        u = ((w >> np.uint64(8)).astype(np.float64) + 0.5) / 2.0 ** 24
        return -np.log(-np.log(u))

    tiles = [(t * 32, min(V, t * 32 + 32)) for t in range((V + 31) // 32)]
    for b in range(B):
        zb = z[b, 0].astype(np.float64)
        lse_t = np.array([np.log(np.exp(zb[a:c]).sum()) for a, c in tiles])
        s1 = lse_t + g(3, b, range(len(tiles)))
        t = int(np.argmax(s1))
        a, c = tiles[t]
        s2 = zb[a:c] + g(0, b, range(a, c))
        assert out["x"][b, 0] == a + int(np.argmax(s2))
        gap1 = np.sort(s1)[-1] - np.sort(s1)[-2]
        gap2 = np.sort(s2)[-1] - np.sort(s2)[-2]
        assert out["margin"][b, 0] == pytest.approx(min(gap1, gap2), abs=1e-9)


def test_temperature_scales_logits():
    """T = 0.5 samples from softmax(2 z); lse is logsumexp(z / T)."""
    z = np.array([0.0, 0.5, -0.5, 1.0], np.float32)
    B = 200_000
    U = _broadcast_draft_inputs([z], B)
    W = np.zeros((4, 1), np.float32)
    out = oracle.draft(U, W, W, np.zeros(B), np.full(B, 0.5, np.float32), seed=8, round_id=1)
    zz = 2.0 * z.astype(np.float64)
    lse = np.log(np.exp(zz).sum())
    np.testing.assert_allclose(out["lse"][:, 0], lse, rtol=1e-14)
    chi2, dof = _chi2(np.bincount(out["x"][:, 0], minlength=4), np.exp(zz - lse))
    assert chi2 < _chi2_crit(dof)


def test_greedy_draft_lowest_index_ties():
    U = np.array([[[0.5, 2.0, 2.0, -1.0]], [[3.0, 3.0, 3.0, 3.0]]], np.float32)
    W = np.zeros((4, 1), np.float32)
    out = oracle.draft(U, W, W, np.zeros(2), np.zeros(2, np.float32), seed=0, round_id=0)
    assert out["x"][:, 0].tolist() == [1, 0]
    assert out["qx"][:, 0].tolist() == [1.0, 1.0]
    assert out["margin"][0, 0] == 0.0
    assert out["lse"][0, 0] == 2.0


def test_markov_bias_is_gathered_row_times_w2():
    """The bias of token v after token a is sum_i W1[a, i] W2[v, i]: with T = 0
    and zero base logits the greedy draft is argmax_v of that bilinear form;
    a transposed operand or a wrong gather row picks a different token."""
    rng = np.random.default_rng(5)
    V, r = 7, 3
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    W2 = rng.standard_normal((V, r)).astype(np.float32)
    for a in range(V):
        U = np.zeros((1, 1, V), np.float32)
        out = oracle.draft(U, W1, W2, np.array([a]), np.zeros(1, np.float32), seed=0, round_id=0)
        bias = W2.astype(np.float64) @ W1[a].astype(np.float64)
        assert out["x"][0, 0] == int(np.argmax(bias))
        assert out["lse"][0, 0] == pytest.approx(bias.max(), abs=1e-12)


# ---------------------------------------------------------------- verify

def _toy_verify(q, p, B, seed=21, gamma=1, ell=None, T=1.0):
    """Feed the section-05 toy through draft + verify: U = ln q, W2 = 0,
    target rows ln p at every position (bonus row included)."""
    q = np.asarray(q, np.float64)
    p = np.asarray(p, np.float64)
    V = len(q)
    W = np.zeros((V, 1), np.float32)
    Urow = np.log(q).astype(np.float32)
    U = _broadcast_draft_inputs([Urow] * gamma, B)
    temp = np.full(B, T, np.float32)
    anchor = np.zeros(B, np.int32)
    d = oracle.draft(U, W, W, anchor, temp, seed=seed, round_id=0)
    ell = np.full(B, gamma if ell is None else ell, np.int32)
    nrows = int((1 + ell).sum())
    target = np.ascontiguousarray(np.broadcast_to(np.log(p).astype(np.float32), (nrows, V)))
    v = oracle.verify(target, ell, U, W, W, anchor, d["x"], temp, seed=seed, round_id=0)
    return d, v


def test_exact_sampling_toy_section05():
    g = _golden("exact_sampling_toy.txt")
    q = [float(t) for t in g["q"]]
    p = [float(t) for t in g["p"]]
    acc_expected = float(g["acceptance"][0])
    resid = [float(t) for t in g["residual_normalised"]]
    kept = [float(t) for t in g["accepted_mass"]]
    S_expected = float(g["residual_mass"][0])
    # the fixture's own arithmetic
    np.testing.assert_allclose(np.minimum(p, q), kept, atol=1e-12)
    B = 1_000_000
    d, v = _toy_verify(q, p, B)
    x1 = d["x"][:, 0]
    n = v["n"]
    acc = (n == 1).mean()
    assert abs(acc - acc_expected) < 3 * math.sqrt(acc_expected * (1 - acc_expected) / B)
    # draws of the draft follow q
    chi2, dof = _chi2(np.bincount(x1, minlength=3), q)
    assert chi2 < _chi2_crit(dof)
    # accepted mass per token: P(x1 = v and accepted) = min(p, q)
    acc_counts = np.bincount(x1[n == 1], minlength=3) / B
    np.testing.assert_allclose(acc_counts, kept, atol=4 * math.sqrt(0.25 / B))
    # residual draws follow (0, 0.6, 0.4); token 0 never comes out of the residual
    y_rej = v["tokens"][n == 0, 0]
    chi2, dof = _chi2(np.bincount(y_rej, minlength=3), resid)
    assert chi2 < _chi2_crit(dof)
    # residual mass at each rejection is 0.20
    np.testing.assert_allclose(v["resid"][n == 0], S_expected, atol=1e-6)
    # the first emitted token follows p (losslessness)
    chi2, dof = _chi2(np.bincount(v["tokens"][:, 0], minlength=3), p)
    assert chi2 < 13.82 and dof == 2
    # diag: p(x) and min(1, p/q) at the tested position (the oracle reads the
    # logits ln p, ln q as float32, so compare at float32 input precision)
    pd = np.asarray(p)[x1]
    np.testing.assert_allclose(v["diag"][:, 0, 0], pd, rtol=1e-6)
    np.testing.assert_allclose(v["diag"][:, 0, 1], np.minimum(1.0, pd / np.asarray(q)[x1]), rtol=1e-6)
    # all accepted -> bonus token drawn from p (row 2), also lossless
    bonus = v["tokens"][n == 1, 1]
    chi2, dof = _chi2(np.bincount(bonus, minlength=3), p)
    assert chi2 < _chi2_crit(dof)


def test_q_equals_p_accepts_everything():
    q = [0.5, 0.3, 0.2]
    B = 100_000
    for gamma in (1, 3):
        d, v = _toy_verify(q, q, B, gamma=gamma, seed=4)
        assert np.all(v["n"] == gamma)
        assert np.all(v["tokens"][:, :gamma] == d["x"])
        assert np.all(v["tokens"][:, gamma] >= 0)
        assert np.all(v["resid"] == -1.0)
        np.testing.assert_allclose(v["diag"][:, :gamma, 1], 1.0)


def test_acceptance_equals_one_minus_tv():
    """Per-position acceptance probability = sum min(p, q) = 1 - TV(p, q);
    the residual mass S at a rejection equals TV(p, q)."""
    rng = np.random.default_rng(17)
    V = 8
    q = rng.dirichlet(np.ones(V))
    p = rng.dirichlet(np.ones(V))
    # round the distributions through float32 logits, as the oracle reads them
    q = np.exp(np.log(q).astype(np.float32).astype(np.float64))
    q /= q.sum()
    p = np.exp(np.log(p).astype(np.float32).astype(np.float64))
    p /= p.sum()
    tv = 0.5 * np.abs(p - q).sum()
    alpha = np.minimum(p, q).sum()
    assert alpha == pytest.approx(1 - tv, abs=1e-12)
    B = 200_000
    d, v = _toy_verify(q, p, B, seed=99)
    acc = (v["n"] == 1).mean()
    assert abs(acc - alpha) < 4 * math.sqrt(alpha * (1 - alpha) / B)
    np.testing.assert_allclose(v["resid"][v["n"] == 0], tv, rtol=1e-9)


def test_expected_accepted_length_closed_form():
    """With W2 = 0 the draft at each position ignores the prefix, so
    E[n] = sum_{j<=ell} prod_{i<=j} alpha_i with alpha_i = sum min(p_i, q_i)."""
    rng = np.random.default_rng(23)
    V, gamma, B = 6, 4, 200_000
    qs = [rng.dirichlet(np.ones(V) * 2) for _ in range(gamma)]
    ps = [rng.dirichlet(np.ones(V) * 2) for _ in range(gamma + 1)]
    Urows = np.log(np.array(qs)).astype(np.float32)
    W = np.zeros((V, 1), np.float32)
    U = _broadcast_draft_inputs(Urows, B)
    temp = np.ones(B, np.float32)
    anchor = np.zeros(B, np.int32)
    d = oracle.draft(U, W, W, anchor, temp, seed=31, round_id=2)
    ell = np.full(B, gamma, np.int32)
    trows = np.log(np.array(ps)).astype(np.float32)
    target = np.ascontiguousarray(np.tile(trows, (B, 1)))
    v = oracle.verify(target, ell, U, W, W, anchor, d["x"], temp, seed=31, round_id=2)
    qf = np.exp(Urows.astype(np.float64))
    qf /= qf.sum(1, keepdims=True)
    pf = np.exp(trows.astype(np.float64))
    pf /= pf.sum(1, keepdims=True)
    alpha = np.minimum(pf[:gamma], qf).sum(1)
    en = np.cumprod(alpha).sum()
    n = v["n"].astype(np.float64)
    assert abs(n.mean() - en) < 4 * n.std() / math.sqrt(B)
    # P(n >= j) = prod_{i<=j} alpha_i
    for j in range(1, gamma + 1):
        pj = np.prod(alpha[:j])
        assert abs((v["n"] >= j).mean() - pj) < 4 * math.sqrt(pj * (1 - pj) / B) + 1e-12


def test_multi_position_losslessness_with_markov_head():
    """With a prefix-dependent draft (nonzero Markov head) the token emitted at
    position k, among rounds that reach k, follows the target row p_k."""
    rng = np.random.default_rng(41)
    V, r, gamma, B = 6, 2, 3, 300_000
    W1 = (rng.standard_normal((V, r)) * 0.8).astype(np.float32)
    W2 = (rng.standard_normal((V, r)) * 0.8).astype(np.float32)
    Urows = rng.standard_normal((gamma, V)).astype(np.float32)
    U = _broadcast_draft_inputs(Urows, B)
    temp = np.ones(B, np.float32)
    anchor = np.full(B, 2, np.int32)
    d = oracle.draft(U, W1, W2, anchor, temp, seed=5, round_id=3)
    trows = (Urows[0] + rng.standard_normal((gamma + 1, V))).astype(np.float32)
    ell = np.full(B, gamma, np.int32)
    target = np.ascontiguousarray(np.tile(trows, (B, 1)))
    v = oracle.verify(target, ell, U, W1, W2, anchor, d["x"], temp, seed=5, round_id=3)
    pf = np.exp(trows.astype(np.float64))
    pf /= pf.sum(1, keepdims=True)
    for k in range(1, gamma + 2):
        reach = v["n"] >= k - 1
        tok = v["tokens"][reach, k - 1]
        chi2, dof = _chi2(np.bincount(tok, minlength=V), pf[k - 1])
        assert chi2 < _chi2_crit(dof), (k, chi2)


def test_ell_zero_emits_one_token_from_p1():
    q = [0.6, 0.3, 0.1]
    p = [0.2, 0.2, 0.6]
    B = 100_000
    d, v = _toy_verify(q, p, B, gamma=2, ell=0, seed=12)
    assert np.all(v["n"] == 0)
    assert np.all(v["tokens"][:, 1:] == -1)
    chi2, dof = _chi2(np.bincount(v["tokens"][:, 0], minlength=3), p)
    assert chi2 < _chi2_crit(dof)


def test_bonus_draw_skips_zero_mass_tokens():
    """Zero-probability tokens are never drawn by the bonus / resample draw,
    and the draw frequencies follow the mass, across tile boundaries."""
    logits = np.full(70, NEG, np.float32)
    logits[[1, 4, 6, 31, 32, 50, 69]] = [0.0, 1.0, -0.5, 0.3, -1.0, 0.7, 0.1]
    p = np.exp(np.where(np.isinf(logits), -np.inf, logits).astype(np.float64))
    p /= p.sum()
    B = 200_000
    V = len(logits)
    W = np.zeros((V, 1), np.float32)
    U = _broadcast_draft_inputs([np.zeros(V, np.float32)], B)
    temp = np.ones(B, np.float32)
    d = oracle.draft(U, W, W, np.zeros(B, np.int32), temp, seed=2, round_id=0)
    ell = np.zeros(B, np.int32)
    target = np.ascontiguousarray(np.broadcast_to(logits, (B, V)))
    v = oracle.verify(target, ell, U, W, W, np.zeros(B, np.int32), d["x"], temp, seed=2, round_id=0)
    chi2, dof = _chi2(np.bincount(v["tokens"][:, 0], minlength=V), p)
    assert chi2 < _chi2_crit(dof)


def test_bonus_draw_brute_force_small_vocab():
    """For V <= 32 (one tile), every bonus token is the entry maximising
    log p(v) + G(v) with G = -log(-log u) of the stream-2 word of
    (position 1, request, v), recomputed here with numpy from the raw words."""
    rng = np.random.default_rng(77)
    for V in (1, 2, 3, 5, 16):
        logits = rng.standard_normal(V).astype(np.float32)
        B = 500
        W = np.zeros((V, 1), np.float32)
        U = _broadcast_draft_inputs([np.zeros(V, np.float32)], B)
        temp = np.ones(B, np.float32)
        seed = 100 + V
        d = oracle.draft(U, W, W, np.zeros(B, np.int32), temp, seed=seed, round_id=4)
        target = np.ascontiguousarray(np.broadcast_to(logits, (B, V)))
        v = oracle.verify(target, np.zeros(B, np.int32), U, W, W, np.zeros(B, np.int32), d["x"], temp,
                          seed=seed, round_id=4)
        z = logits.astype(np.float64)
        for b in range(B):
            words = np.array([oracle.random_word(seed, 4, 2, 1, b, i) for i in range(V)], np.uint64)
            u = ((words >> np.uint64(8)).astype(np.float64) + 0.5) / 2.0 ** 24
            assert v["tokens"][b, 0] == int(np.argmax(z - np.log(-np.log(u))))


def test_residual_draw_follows_residual_across_tiles():
    """After a rejection, y follows r = max(p - q, 0) / sum(...) over a
    vocabulary of several tiles (chi-square), and every emitted first token
    follows p."""
    rng = np.random.default_rng(31)
    V = 80
    q = rng.dirichlet(np.ones(V))
    p = rng.dirichlet(np.ones(V))
    B = 400_000
    d, v = _toy_verify(q, p, B, seed=13)
    qf = np.exp(np.log(q).astype(np.float32).astype(np.float64))
    qf /= qf.sum()
    pf = np.exp(np.log(p).astype(np.float32).astype(np.float64))
    pf /= pf.sum()
    r = np.maximum(pf - qf, 0)
    r /= r.sum()
    rej = v["n"] == 0
    counts = np.bincount(v["tokens"][rej, 0], minlength=V)
    assert np.all(counts[r == 0] == 0)
    e = rej.sum() * r
    keep = e >= 5
    c2 = (((counts[keep] - e[keep]) ** 2) / e[keep]).sum()
    assert c2 < _chi2_crit(int(keep.sum()) - 1)
    counts = np.bincount(v["tokens"][:, 0], minlength=V)
    e = B * pf
    keep = e >= 5
    c2 = (((counts[keep] - e[keep]) ** 2) / e[keep]).sum()
    assert c2 < _chi2_crit(int(keep.sum()) - 1)


def test_residual_draw_uses_position_of_rejection():
    """The resample noise is drawn at the rejected position j: two requests
    that differ only in where they reject get independent draws, and the
    residual draw at j never returns a token with p_j <= q_j."""
    q = np.array([0.70, 0.18, 0.12])
    p = np.array([0.50, 0.30, 0.20])
    B = 20000
    d, v = _toy_verify(q, p, B, gamma=3, seed=8)
    n = v["n"]
    for j in (1, 2, 3):
        rej = n == j - 1
        y = v["tokens"][rej, j - 1]
        assert np.all(y != 0)  # token 0 has p < q: no residual mass


def test_greedy_verify_is_longest_matching_prefix():
    """T = 0: n = length of the longest prefix where the draft equals the
    target argmax, and the emitted token is the target argmax at n + 1."""
    rng = np.random.default_rng(9)
    V, gamma, B = 12, 5, 400
    W1 = rng.standard_normal((V, 2)).astype(np.float32)
    W2 = rng.standard_normal((V, 2)).astype(np.float32)
    U = rng.standard_normal((B, gamma, V)).astype(np.float32)
    temp = np.zeros(B, np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    d = oracle.draft(U, W1, W2, anchor, temp, seed=0, round_id=0)
    x = d["x"]
    ell = rng.integers(0, gamma + 1, B).astype(np.int32)
    rows, tam = [], []
    for b in range(B):
        for k in range(ell[b] + 1):
            t = rng.standard_normal(V).astype(np.float32)
            if k < ell[b] and rng.random() < 0.7:  # make the draft match often
                t[x[b, k]] = t.max() + 1.0
            rows.append(t)
    target = np.array(rows, np.float32)
    v = oracle.verify(target, ell, U, W1, W2, anchor, x, temp, seed=0, round_id=0)
    off = 0
    for b in range(B):
        am = [int(np.argmax(target[off + k])) for k in range(ell[b] + 1)]
        n = 0
        while n < ell[b] and x[b, n] == am[n]:
            n += 1
        assert v["n"][b] == n
        assert v["tokens"][b, :n].tolist() == x[b, :n].tolist()
        assert v["tokens"][b, n] == am[n]
        assert np.all(v["tokens"][b, n + 1:] == -1)
        off += ell[b] + 1


def test_verify_rejects_bad_lengths():
    V = 3
    W = np.zeros((V, 1), np.float32)
    U = np.zeros((1, 2, V), np.float32)
    with pytest.raises(ValueError):
        oracle.verify(np.zeros((4, V), np.float32), np.array([3]), U, W, W, np.zeros(1), np.zeros((1, 2)),
                      np.ones(1, np.float32), seed=0, round_id=0)
