"""Pins for the oracle's RNN-head draft (page "DSpark：DeepSeek 线上跑的投机解码..."
(marsggbo.github.io), section 3.2, the RNN Head: a GRU-like state s_k over
the block, z = [s_{k-1}, W1[x_{k-1}], h_k], (gate, candidate, output) =
Wgco z, s_k = g s_{k-1} + (1 - g) tanh(candidate), B_k = W2 tanh(output)).

Each test fixes the result by something outside the RNN code: torch's
bfloat16 conversion, the Markov-head draft (already pinned against the pages'
examples and sampling identities) for configurations in which the RNN head
reduces to a Markov head, closed forms of the state recurrence, and the
rejection rule's losslessness.
"""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-40, 38, 4000),
                        rng.standard_normal(1000)]).astype(np.float32)
    # exact halfway cases: a bfloat16 value plus half its last place
    base = (rng.standard_normal(500).astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000))
    halves = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, halves, np.float32([0.0, -0.0, 1.0, 3.3895314e38, 1e-42])])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_round(float(v)) for v in x])
    np.testing.assert_array_equal(got, want)


def _rnn_inputs(B, gamma, V, r, d, seed):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 1.5, (B, gamma, V)).astype(np.float32)
    W1 = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    W2 = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    h = rng.normal(0, 1.0, (B, gamma, d)).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    temp = np.where(np.arange(B) % 3 == 0, 0.0, 1.0).astype(np.float32)
    return U, W1, W2, h, anchor, temp


def test_zero_head_weights_draw_from_the_base_logits():
    """Wgco = 0: every gate is sigmoid(0) = 1/2 and every tanh 0, so the state
    stays 0 and the bias vanishes: the draft is the Markov draft with W2 = 0."""
    B, gamma, V, r, d = 12, 4, 70, 4, 6
    U, W1, W2, h, anchor, temp = _rnn_inputs(B, gamma, V, r, d, 2)
    Wgco = np.zeros((3 * r, 2 * r + d), np.float32)
    o = oracle.draft_rnn(U, W1, W2, Wgco, h, anchor, temp, seed=3, round_id=1)
    m = oracle.draft(U, W1, np.zeros_like(W2), anchor, temp, seed=3, round_id=1)
    for k in ("x", "lse", "qx", "margin"):
        np.testing.assert_array_equal(o[k], m[k])
    assert np.all(o["state"] == 0) and np.all(o["e"] == 0)


def test_output_gate_reading_the_embedding_is_a_markov_head():
    """An output gate that reads only the W1 block of z through the identity
    gives e_k = bf16(tanh(W1[x_{k-1}])): the RNN draft equals the Markov draft
    whose embedding rows are bf16(tanh(W1)).  Any other column order of the
    concatenation, or rows of Wgco taken in another gate order, breaks it."""
    B, gamma, V, r, d = 16, 5, 90, 8, 16
    U, W1, W2, h, anchor, temp = _rnn_inputs(B, gamma, V, r, d, 4)
    rng = np.random.default_rng(5)
    Wgco = np.zeros((3 * r, 2 * r + d), np.float32)
    Wgco[:r] = rng.normal(0, 0.5, (r, 2 * r + d))        # gate: anything
    Wgco[r:2 * r] = rng.normal(0, 0.5, (r, 2 * r + d))   # candidate: anything
    Wgco[2 * r:, r:2 * r] = np.eye(r)                    # output = W1[x_{k-1}]
    o = oracle.draft_rnn(U, W1, W2, Wgco, h, anchor, temp, seed=8, round_id=0)
    W1m = np.vectorize(lambda v: oracle.bf16_round(math.tanh(v)))(W1.astype(np.float64)).astype(np.float32)
    m = oracle.draft(U, W1m, W2, anchor, temp, seed=8, round_id=0)
    for k in ("x", "lse", "qx", "margin"):
        np.testing.assert_allclose(o[k], m[k], rtol=0, atol=1e-12, err_msg=k)
    prev = np.concatenate([anchor[:, None], o["x"][:, :-1]], axis=1)
    np.testing.assert_array_equal(o["e"], W1m[prev].astype(np.float64))


def test_state_closed_form_with_constant_gates():
    """Gates fed by one constant coordinate of h only: y_gate = a, y_cand = c
    for every position, so s_k = tanh(c) (1 - sigmoid(a)^k)."""
    B, gamma, V, r, d = 3, 7, 40, 4, 2
    U, W1, W2, h, anchor, temp = _rnn_inputs(B, gamma, V, r, d, 6)
    h[:] = 0.0
    h[:, :, 1] = 1.0
    a = np.array([0.3, -1.2, 2.0, 0.0])
    c = np.array([0.7, -0.4, 1.5, -2.0])
    # a and c as bfloat16-exact float32 weights: h = 1 enters exactly
    a = np.array([oracle.bf16_round(v) for v in a])
    c = np.array([oracle.bf16_round(v) for v in c])
    Wgco = np.zeros((3 * r, 2 * r + d), np.float32)
    Wgco[:r, 2 * r + 1] = a
    Wgco[r:2 * r, 2 * r + 1] = c
    o = oracle.draft_rnn(U, W1, W2, Wgco, h, anchor, temp, seed=1, round_id=0)
    sig = 1.0 / (1.0 + np.exp(-a))
    want = np.tanh(c) * (1.0 - sig ** gamma)
    np.testing.assert_allclose(o["state"], np.broadcast_to(want, (B, r)), rtol=1e-14, atol=1e-15)
    assert np.all(o["e"] == 0)  # the output gate sees nothing


def test_state_feeds_the_next_position():
    """An output gate that reads the state block: e_1 = 0 (s_0 = 0), and
    e_k = bf16(tanh(beta * bf16(s_{k-1}))) with s_k from a constant candidate
    and a gate of 1/2: s_k = (1 - 2^-k) tanh(c)."""
    B, gamma, V, r, d = 2, 4, 30, 4, 1
    U, W1, W2, h, anchor, temp = _rnn_inputs(B, gamma, V, r, d, 7)
    h[:] = 1.0
    beta, c = 2.0, 0.75
    Wgco = np.zeros((3 * r, 2 * r + d), np.float32)
    Wgco[r:2 * r, 2 * r] = c
    Wgco[2 * r:, :r] = beta * np.eye(r)
    o = oracle.draft_rnn(U, W1, W2, Wgco, h, anchor, temp, seed=2, round_id=0)
    assert np.all(o["e"][:, 0] == 0)
    for k in range(2, gamma + 1):
        s_prev = (1.0 - 2.0 ** -(k - 1)) * math.tanh(c)
        want = oracle.bf16_round(math.tanh(beta * oracle.bf16_round(s_prev)))
        np.testing.assert_array_equal(o["e"][:, k - 1], want)
    np.testing.assert_allclose(o["state"], (1.0 - 2.0 ** -gamma) * math.tanh(c), rtol=1e-14)


def test_verify_with_head_rows_equal_to_the_embedding_is_the_markov_verify():
    """Verification that reads the head's rows E[b][k-1] = W1[x_{k-1}] is the
    Markov-head verification, bit for bit."""
    B, gamma, V, r = 20, 4, 60, 4
    U, W1, W2, _, anchor, temp = _rnn_inputs(B, gamma, V, r, 1, 9)
    d = oracle.draft(U, W1, W2, anchor, temp, seed=4, round_id=0)
    ell = np.random.default_rng(3).integers(0, gamma + 1, B).astype(np.int32)
    target = np.random.default_rng(4).normal(0, 1.5, (int((1 + ell).sum()), V)).astype(np.float32)
    prev = np.concatenate([anchor[:, None], d["x"][:, :-1]], axis=1)
    E = W1[prev]
    a = oracle.verify(target, ell, U, W1, W2, anchor, d["x"], temp, seed=4, round_id=0)
    b = oracle.verify(target, ell, U, np.zeros_like(W1), W2, anchor, d["x"], temp, seed=4, round_id=0, head_rows=E)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    aa = oracle.acceptance(target, ell, U, W1, W2, anchor, d["x"], temp)
    ab = oracle.acceptance(target, ell, U, np.zeros_like(W1), W2, anchor, d["x"], temp, head_rows=E)
    np.testing.assert_array_equal(aa, ab)


def test_rnn_round_is_lossless():
    """Draft with the RNN head, verify against its rows: among the rounds that
    reach position k, the token emitted there follows the target row p_k (the
    target rows here do not depend on the prefix), whatever the head does."""
    from scipy.stats import chi2
    B, gamma, V, r, d = 120_000, 2, 5, 2, 2
    rng = np.random.default_rng(11)
    Urow = rng.normal(0, 1.0, (gamma, V)).astype(np.float32)
    U = np.ascontiguousarray(np.broadcast_to(Urow, (B, gamma, V)))
    W1 = rng.normal(0, 0.8, (V, r)).astype(np.float32)
    W2 = rng.normal(0, 0.8, (V, r)).astype(np.float32)
    Wgco = rng.normal(0, 0.8, (3 * r, 2 * r + d)).astype(np.float32)
    h = np.ascontiguousarray(np.broadcast_to(rng.normal(0, 1, (gamma, d)).astype(np.float32), (B, gamma, d)))
    anchor = np.full(B, 1, np.int32)
    temp = np.ones(B, np.float32)
    o = oracle.draft_rnn(U, W1, W2, Wgco, h, anchor, temp, seed=6, round_id=0)
    trow = rng.normal(0, 1.0, (gamma + 1, V)).astype(np.float32)
    ell = np.full(B, gamma, np.int32)
    target = np.ascontiguousarray(np.broadcast_to(trow, (B, gamma + 1, V)).reshape(-1, V))
    v = oracle.verify(target, ell, U, W1, W2, anchor, o["x"], temp, seed=6, round_id=0, head_rows=o["e"])
    for pos in range(gamma + 1):  # the token at position pos + 1 of the rounds that reach it
        p = np.exp(trow[pos].astype(np.float64))
        p /= p.sum()
        tok = v["tokens"][v["n"] >= pos, pos]
        counts = np.bincount(tok, minlength=V)
        n = len(tok)
        stat = ((counts - n * p) ** 2 / (n * p)).sum()
        assert stat < chi2.ppf(1 - 1e-3, V - 1), (pos, stat)
