"""GPU parity of the RNN-head variant (page "DSpark：DeepSeek 线上跑的投机解码..."
(marsggbo.github.io), section 3.2, the RNN Head) through the C ABI, against
the fp64 oracle on the same seeded inputs and Philox streams.

Draft decisions are compared as for the Markov head (eligible requests: every
Gumbel margin > 1e-3, exact tokens; probabilities within 1e-4).  The head's
rows e_k are bfloat16 on both sides, rounded from float32 on the GPU and from
double in the oracle, so an element may differ by one bfloat16 step where
the two straddle a rounding boundary, plus the float32 gate product's
absolute error and, after position 1, the effect of a state entry that the
two sides round to neighbouring bfloat16 values (bounds in _check_rows);
they are compared where the drafts agree on x_1..x_{k-1}.  The state s_gamma
agrees within 2e-3 for the same reason (measured: 1.7e-4 at r = 256,
d = 1024; 1e-7 where no entry rounds apart).
"""
import numpy as np
import pytest

import oracle
import synth_inputs as S
from roundkit import (ACCEPT_MARGIN, DRAFT_MARGIN, GREEDY_MARGIN, PICK_MARGIN, PROB_TOL, np_of, packed_subset,
                      to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import draft_sampling_verification_02_amd as ds  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _rnn_case(B, gamma, V, r, d, seed, greedy_every=0, w_std=0.05):
    cfg = S.Config("custom", B=B, gamma=gamma, V=V, r=r, wdtype="bf16", w_std=w_std, u_std=3.0, noise_std=1.0,
                   seed=seed, greedy_every=greedy_every)
    rnd = S.make_round(cfg)
    h, _ = S.confidence_head_inputs(cfg, d)
    bits, Wg = S.rnn_head_weights(cfg, d)
    return cfg, rnd, h, bits, Wg


def _dev_rnn(rnd, h, bits):
    dev = to_device(rnd)
    dev["hidden"] = torch.from_numpy(h).cuda()
    dev["Wgco"] = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return dev


def _gpu_draft_rnn(dev, seed, rid, state=True):
    return ds.dspark_draft_sample_rnn(dev["U"], dev["W1"], dev["W2"], dev["Wgco"], dev["anchor"],
                                      dev["temperature"], dev["hidden"], seed, rid, margin=True, state=state)


def _e_of(t):
    return t.float().cpu().numpy().astype(np.float64)


def _prefix_agree(gx, ox):
    eq = gx == ox
    agree = np.ones_like(eq)
    agree[:, 1:] = np.cumprod(eq[:, :-1], axis=1).astype(bool)
    return agree


def _check_rows(ge, oe, ok, tag):
    """e rows [B, gamma, r].  Position 1 (s_0 = 0): the GPU's tanh(y) carries
    only the float32 gate product's absolute error (<= 1e-5 here), and both
    sides round to bfloat16, so they differ by at most one bfloat16 step of
    the value plus that error.  Later positions also take s_{k-1} rounded to
    bfloat16, where the float32 and double states can round to neighbours:
    one such entry moves y by |w| * 2^-8 * |s| <= 4e-4 (|w| within four
    standard deviations of (2r + d)^-1/2, |s| < 1), a few of them a row, so
    the bound there is one step plus 1e-3."""
    ok1 = ok.copy()
    ok1[:, 1:] = False
    okn = ok.copy()
    okn[:, 0] = False
    for sel, extra, what in ((ok1, 1e-5, "k=1"), (okn, 1e-3, "k>1")):
        diff = np.abs(ge[sel] - oe[sel])
        if not diff.size:
            continue
        step = np.maximum(np.abs(oe[sel]), 2.0 ** -126) * 2.0 ** -7
        bad = diff > step + extra
        assert not bad.any(), f"{tag} {what}: e off by {diff[bad].max():.3e} at |e| = {np.abs(oe[sel][bad]).min():.3e}"
        _say(f"[{tag}] e rows {what}: {sel.sum()} compared, {float((diff > 0).mean()):.2e} of the entries apart, "
             f"max |de| {diff.max():.2e}")


def _shift_bound(ge, oe, W2, ok):
    """[B, gamma]: the largest logit shift the two sides' e_k differences can
    cause, max_v sum_i |W2[v, i]| |de_i|, at positions whose prefixes agree
    (0 where e_k is the same bits on both sides)."""
    de = np.abs(ge - oe)
    bound = np.zeros(ok.shape)
    for b, k in zip(*np.nonzero(ok & np.any(de > 0, axis=2))):
        idx = np.nonzero(de[b, k])[0]
        bound[b, k] = (np.abs(W2[:, idx].astype(np.float64)) @ de[b, k, idx]).max()
    return bound


def _compare_rnn_draft(gd, od, bound, temperature, tag):
    """Tokens exact where every oracle margin clears 1e-3 plus twice the
    shift the e differences explain (in the units of the draw: logits / T);
    lse and q(x) within 1e-4 plus that shift.  Returns the eligible mask."""
    sampled = temperature > 0
    scale = np.where(sampled, 1.0 / np.where(sampled, temperature, 1.0), 1.0)[:, None]
    shift = bound * scale
    el = np.all(od["margin"] > DRAFT_MARGIN + 2 * shift, axis=1)
    np.testing.assert_array_equal(gd["x"][el], od["x"][el])
    dl = np.abs(gd["lse"] - od["lse"])[el]
    assert np.all(dl <= PROB_TOL + shift[el]), f"{tag}: lse off by {dl.max():.2e}"
    dq = np.abs(gd["qx"] - od["qx"])[el]
    assert np.all(dq <= PROB_TOL + od["qx"][el] * np.expm1(2 * shift[el])), f"{tag}: q(x) off by {dq.max():.2e}"
    mism = np.any(gd["x"] != od["x"], axis=1)
    _say(f"[{tag}] draft: {el.sum()}/{len(el)} eligible, {int(mism[~el].sum())} of the rest differ; "
         f"positions with e apart: {int((bound > 0).sum())}, largest logit shift {bound.max():.2e}; "
         f"max |dlse| {dl.max() if dl.size else 0:.2e}")
    return el


@pytest.mark.parametrize("B,gamma,V,r,d", [
    (1, 4, 1000, 16, 32),
    (5, 3, 17, 16, 0),        # no hidden part; a K step straddles s / W1
    (33, 4, 1003, 32, 64),    # ragged batch and vocabulary
    (40, 5, 2053, 256, 512),  # the headline rank, the per-position product covering h
    (70, 6, 4099, 64, 96),
    (300, 2, 700, 128, 32),   # many request tiles
    # d >= 4r (and gamma >= 2): the h part is precomputed for the whole block
    (40, 5, 2053, 256, 1024), # the headline head shape
    (40, 5, 2053, 256, 2048), # 8 K splits of 256
    (17, 3, 1003, 16, 96),    # 3 splits, each a single 32-wide stage
    (70, 4, 4099, 64, 288),   # 5 splits, the last one 32 wide
    (1, 2, 1000, 16, 96),     # one request: a 2-row product
    (9, 1, 1000, 16, 96),     # gamma 1: not precomputed
])
def test_rnn_draft_parity(B, gamma, V, r, d):
    cfg, rnd, h, bits, Wg = _rnn_case(B, gamma, V, r, d, seed=B * 7 + r + d, greedy_every=4)
    _say(f"[rnn] B={B} gamma={gamma} V={V} r={r} d={d}")
    dev = _dev_rnn(rnd, h, bits)
    g = _gpu_draft_rnn(dev, 33, 5)
    torch.cuda.synchronize()
    od = oracle.draft_rnn(rnd.U, rnd.W1, rnd.W2, Wg, h, rnd.anchor, rnd.temperature, 33, 5)
    gd = {k: np_of(g[k]) for k in ("x", "lse", "qx", "margin")}
    ok = _prefix_agree(gd["x"], od["x"])
    ge = _e_of(g["e"])
    _check_rows(ge, od["e"], np.repeat(ok[:, :, None], r, axis=2), "rnn")
    el = _compare_rnn_draft(gd, od, _shift_bound(ge, od["e"], rnd.W2, ok), rnd.temperature, "rnn")
    assert el.mean() > 0.8
    full = ok[:, -1] & (gd["x"][:, -1] == od["x"][:, -1])
    s_err = np.abs(np_of(g["state"])[full] - od["state"][full]).max() if full.any() else 0.0
    _say(f"[rnn] state: {full.sum()} requests with the whole block equal, max |ds| {s_err:.2e}")
    assert full.any() and s_err < 2e-3  # the neighbouring-rounding effect above, carried through the block


@pytest.mark.parametrize("d", [512, 1024, 4096])
def test_rnn_round_large_batch_config(d):
    """Batch 256, gamma 5, V 129,280, r 256, d 512 (the per-position product
    covers h), 1024 and 4096 (h part precomputed): RNN draft and its verify
    against the oracle on a sample of requests."""
    cfg = S.CONFIGS["large"]
    rnd = S.make_round(cfg)
    h, _ = S.confidence_head_inputs(cfg, d)
    bits, Wg = S.rnn_head_weights(cfg, d)
    ell = np.full(cfg.B, cfg.gamma, np.int32)
    target = rnd.target_packed(ell)
    _say(f"[rnn-large] B={cfg.B} V={cfg.V} d={d}")
    dev = _dev_rnn(rnd, h, bits)
    g = _gpu_draft_rnn(dev, cfg.seed, 0)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    v = ds.dspark_verify_rnn(td, ed, dev["U"], g["e"], dev["W2"], dev["anchor"], g["x"], g["lse"], g["qx"],
                             dev["temperature"], cfg.seed, 0, diag=True, resid=True)
    torch.cuda.synchronize()
    assert ds.dspark_verify_check(v["workspace"]) == 0
    rows = np.arange(cfg.B)
    U, anchor, temp = rnd.U[rows], rnd.anchor[rows], rnd.temperature[rows]
    od = oracle.draft_rnn(U, rnd.W1, rnd.W2, Wg, h[rows], anchor, temp, cfg.seed, 0, req_ids=rows.astype(np.int32))
    sub = packed_subset(target, ell, rows)
    ov = oracle.verify(sub, ell[rows], U, rnd.W1, rnd.W2, anchor, od["x"], temp, cfg.seed, 0,
                       req_ids=rows.astype(np.int32), head_rows=od["e"])
    gd = {k: np_of(g[k])[rows] for k in ("x", "lse", "qx", "margin")}
    gv = {k: np_of(v[k])[rows] for k in ("n", "tokens", "diag", "resid")}
    ok = _prefix_agree(gd["x"], od["x"])
    ge = _e_of(g["e"])[rows]
    _check_rows(ge, od["e"], np.repeat(ok[:, :, None], cfg.r, axis=2), "rnn-large")
    bound = _shift_bound(ge, od["e"], rnd.W2, ok)
    el = _compare_rnn_draft(gd, od, bound, temp, "rnn-large")
    # verify: the accept tests and the draw must clear their margins plus the
    # relative change of q the shift allows; then n and tokens are exact
    rel = np.expm1(2 * bound)  # T = 1 or greedy here
    for i in range(len(rows)):
        if not el[i]:
            continue
        n, L = ov["n"][i], ell[rows][i]
        tested = min(n + 1, L)
        thr = ACCEPT_MARGIN if temp[i] > 0 else GREEDY_MARGIN
        if np.any(ov["accept_margin"][i, :tested] <= thr + 2 * rel[i, :tested]):
            el[i] = False
            continue
        pthr = PICK_MARGIN if temp[i] > 0 else GREEDY_MARGIN
        if not ov["pick_margin"][i] > pthr + 2 * rel[i].max():
            el[i] = False
    np.testing.assert_array_equal(gv["n"][el], ov["n"][el])
    np.testing.assert_array_equal(gv["tokens"][el], ov["tokens"][el])
    dg, do = gv["diag"][el], ov["diag"][el]
    tested = ~np.isnan(do)
    assert np.array_equal(np.isnan(dg), ~tested)
    # column 0 is p(x), which does not involve q; column 1 is min(1, p/q)
    relx = np.concatenate([rel[el], np.zeros((el.sum(), 1))], axis=1)
    lim = PROB_TOL + relx[:, :, None] * np.abs(do) * np.array([0.0, 1.0])
    assert np.all(np.abs(dg - do)[tested] <= lim[tested])
    assert np.all(np.abs(gv["resid"][el] - ov["resid"][el]) <= PROB_TOL + 2 * rel[el].max(initial=0.0))
    _say(f"[rnn-large] verify: {el.sum()}/{len(rows)} eligible, n differs on {int((gv['n'] != ov['n']).sum())}")
    assert el.sum() >= len(rows) // 2


def test_rnn_verify_with_embedding_rows_is_the_markov_verify():
    """dspark_verify_rnn fed the rows W1[x_{k-1}] gives dspark_verify's
    outputs bit for bit (same kernels, rows addressed per position)."""
    B, gamma, V, r = 48, 4, 3001, 64
    cfg = S.Config("custom", B=B, gamma=gamma, V=V, r=r, wdtype="bf16", w_std=0.05, u_std=3.0, noise_std=1.0,
                   seed=12, greedy_every=5)
    rnd = S.make_round(cfg)
    ell = np.random.default_rng(3).integers(0, gamma + 1, B).astype(np.int32)
    target = rnd.target_packed(ell)
    dev = to_device(rnd)
    d = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], 4, 2)
    prev = torch.cat([dev["anchor"][:, None].long(), d["x"][:, :-1].long()], dim=1)
    rows = dev["W1"][prev].contiguous()
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    a = ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"], d["qx"],
                         dev["temperature"], 4, 2, diag=True, resid=True)
    b = ds.dspark_verify_rnn(td, ed, dev["U"], rows, dev["W2"], dev["anchor"], d["x"], d["lse"], d["qx"],
                             dev["temperature"], 4, 2, diag=True, resid=True)
    aa = ds.dspark_acceptance(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"],
                              dev["temperature"])
    ab = ds.dspark_acceptance_rnn(td, ed, dev["U"], rows, dev["W2"], dev["anchor"], d["x"], d["lse"],
                                  dev["temperature"])
    torch.cuda.synchronize()
    for k in ("n", "tokens", "offsets", "diag", "resid"):
        np.testing.assert_array_equal(np_of(a[k]), np_of(b[k]), err_msg=k)
    np.testing.assert_array_equal(np_of(aa), np_of(ab))


def test_rnn_acceptance_parity():
    B, gamma, V, r, d = 30, 4, 1500, 32, 64
    cfg, rnd, h, bits, Wg = _rnn_case(B, gamma, V, r, d, seed=21, greedy_every=3)
    ell = np.random.default_rng(2).integers(0, gamma + 1, B).astype(np.int32)
    target = rnd.target_packed(ell)
    dev = _dev_rnn(rnd, h, bits)
    g = _gpu_draft_rnn(dev, 9, 1, state=False)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    alpha = np_of(ds.dspark_acceptance_rnn(td, ed, dev["U"], g["e"], dev["W2"], dev["anchor"], g["x"], g["lse"],
                                           dev["temperature"]))
    torch.cuda.synchronize()
    od = oracle.draft_rnn(rnd.U, rnd.W1, rnd.W2, Wg, h, rnd.anchor, rnd.temperature, 9, 1)
    ao = oracle.acceptance(target, ell, rnd.U, rnd.W1, rnd.W2, rnd.anchor, od["x"], rnd.temperature,
                           head_rows=od["e"])
    gx = np_of(g["x"])
    sampled = rnd.temperature > 0
    ok_s = _prefix_agree(gx, od["x"])
    ok_g = np.cumprod(gx == od["x"], axis=1).astype(bool)
    ok = np.where(sampled[:, None], ok_s, ok_g)
    verified = np.arange(gamma)[None, :] < ell[:, None]
    np.testing.assert_array_equal(np.isnan(alpha), ~verified)
    cmp = ok & verified
    err = np.abs(alpha[cmp] - ao[cmp]).max()
    _say(f"[rnn-alpha] compared {cmp.sum()}/{verified.sum()}; max |dalpha| {err:.2e}")
    assert cmp.sum() >= 0.8 * verified.sum() and err < 1e-4
