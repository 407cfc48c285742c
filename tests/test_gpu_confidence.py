"""GPU parity of the confidence head, the prefix survival products and the
per-position acceptance probability, through the C ABI, against the fp64
oracle on the same seeded inputs.

The head's c_k and a_k depend on the drafted prefix x_1..x_{k-1}, alpha_k on
x_1..x_{k-1} (sampled rows) or x_1..x_k (greedy rows): each is compared at
the positions where the GPU's and the oracle's drafts agree on that prefix
(nearly all of them; the rest are counted).  Probabilities agree within
1e-4; greedy alpha values are exact.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as S
from roundkit import (PROB_TOL, gpu_verify, np_of, oracle_round, packed_subset, to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import draft_sampling_verification_02_amd as ds  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _prefix_agree(gx, ox, through_k=False):
    """[B, gamma] bool: the drafts x_1..x_{k-1} (x_1..x_k with through_k)
    are the same on both sides."""
    eq = gx == ox
    if through_k:
        return np.cumprod(eq, axis=1).astype(bool)
    agree = np.ones_like(eq)
    agree[:, 1:] = np.cumprod(eq[:, :-1], axis=1).astype(bool)
    return agree


def _case(B, gamma, V, r, wdtype, seed, greedy_every=0, ell=None):
    cfg = S.Config("custom", B=B, gamma=gamma, V=V, r=r, wdtype=wdtype, w_std=0.05, u_std=3.0, noise_std=1.0,
                   seed=seed, greedy_every=greedy_every)
    rnd = S.make_round(cfg)
    if ell is None:
        ell = np.random.default_rng(seed + 7).integers(0, gamma + 1, B).astype(np.int32)
    return cfg, rnd, np.asarray(ell, np.int32)


def _gpu_conf(dev, h, w, seed, round_id):
    hd = torch.from_numpy(h).cuda()
    wd = torch.from_numpy(w).cuda()
    return ds.dspark_draft_sample_confidence(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"],
                                             hd, wd, seed, round_id, margin=True)


# ---------------------------------------------------------------- confidence head

@pytest.mark.parametrize("B,gamma,V,r,wdtype,d", [
    (1, 4, 1000, 16, "f32", 64),
    (5, 3, 17, 16, "bf16", 0),          # no hidden part: the W1 half only
    (33, 4, 1003, 32, "bf16", 3),       # scalar loads, d below one wave
    (70, 6, 4099, 64, "f32", 1030),     # scalar loads, d not a multiple of 4
    (40, 5, 2053, 256, "bf16", 1024),   # float4 loads in one batch
    (9, 7, 700, 128, "bf16", 4100),     # float4 loads, several batches and a ragged tail
    (300, 2, 300, 16, "bf16", 8),       # many workgroups of requests
])
def test_confidence_head_parity(B, gamma, V, r, wdtype, d):
    cfg, rnd, _ = _case(B, gamma, V, r, wdtype, seed=B * 13 + d, greedy_every=4)
    h, w = S.confidence_head_inputs(cfg, d)
    _say(f"[conf] B={B} gamma={gamma} V={V} r={r} {wdtype} d={d}")
    dev = to_device(rnd)
    seed, rid = 91, 4
    gc = _gpu_conf(dev, h, w, seed, rid)
    g0 = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, rid,
                                margin=True)
    torch.cuda.synchronize()
    # the sampling outputs are the plain entry point's, bit for bit
    for key in ("x", "lse", "qx", "margin"):
        np.testing.assert_array_equal(np_of(gc[key]), np_of(g0[key]), err_msg=key)
    od = oracle.draft(rnd.U, rnd.W1, rnd.W2, rnd.anchor, rnd.temperature, seed, rid)
    c, a = oracle.confidence(h, w, rnd.W1, rnd.anchor, od["x"])
    ok = _prefix_agree(np_of(gc["x"]), od["x"])
    c_g, a_g = np_of(gc["conf"]), np_of(gc["survival"])
    err_c = np.abs(c_g[ok] - c[ok]).max()
    err_a = np.abs(a_g[ok] - a[ok]).max()
    _say(f"[conf] compared {ok.sum()}/{ok.size} positions; max |dc| {err_c:.2e} |da| {err_a:.2e}")
    assert ok.mean() > 0.9
    assert err_c < PROB_TOL and err_a < PROB_TOL
    # a_k is the device's own running product of its c_k, one float32 multiply a step
    np.testing.assert_allclose(a_g, np.cumprod(c_g.astype(np.float64), axis=1), rtol=1e-6, atol=0)
    assert np.all((c_g > 0) & (c_g < 1))


def test_confidence_head_large_batch_config():
    """Batch 256, gamma 5, V 129,280, r 256, bf16, d 1024, in the bench's
    launch configuration; the oracle checks every request."""
    cfg = S.CONFIGS["large"]
    rnd = S.make_round(cfg)
    h, w = S.confidence_head_inputs(cfg)
    _say(f"[conf-large] B={cfg.B} V={cfg.V} d={h.shape[2]}")
    dev = to_device(rnd)
    gc = _gpu_conf(dev, h, w, cfg.seed, 0)
    torch.cuda.synchronize()
    rows = np.arange(cfg.B)
    U, anchor, temp = rnd.U[rows], rnd.anchor[rows], rnd.temperature[rows]
    od = oracle.draft(U, rnd.W1, rnd.W2, anchor, temp, cfg.seed, 0, req_ids=rows.astype(np.int32))
    c, a = oracle.confidence(h[rows], w, rnd.W1, anchor, od["x"])
    ok = _prefix_agree(np_of(gc["x"])[rows], od["x"])
    c_g, a_g = np_of(gc["conf"]), np_of(gc["survival"])
    _say(f"[conf-large] compared {ok.sum()}/{ok.size}; mean c {c_g.mean():.3f}")
    assert ok.mean() > 0.8
    np.testing.assert_allclose(c_g[rows][ok], c[ok], rtol=0, atol=PROB_TOL)
    np.testing.assert_allclose(a_g[rows][ok], a[ok], rtol=0, atol=PROB_TOL)
    assert np.all((c_g > 0) & (c_g < 1))
    assert np.all(np.diff(a_g, axis=1) <= 0)


# ---------------------------------------------------------------- acceptance probability

def _gpu_alpha(dev, target, ell, d, row_offsets=None):
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    ro = None if row_offsets is None else torch.from_numpy(row_offsets).cuda()
    return ds.dspark_acceptance(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"],
                                dev["temperature"], row_offsets=ro)


def _compare_alpha(alpha_g, gx, ox, alpha_o, temperature, ell, tag):
    sampled = temperature > 0
    ok = np.where(sampled[:, None], _prefix_agree(gx, ox), _prefix_agree(gx, ox, through_k=True))
    verified = np.arange(alpha_o.shape[1])[None, :] < ell[:, None]
    # NaN exactly past ell (on both sides)
    np.testing.assert_array_equal(np.isnan(alpha_g), ~verified)
    np.testing.assert_array_equal(np.isnan(alpha_o), ~verified)
    cmp = ok & verified
    g_s, o_s = alpha_g[cmp & sampled[:, None]], alpha_o[cmp & sampled[:, None]]
    g_g, o_g = alpha_g[cmp & ~sampled[:, None]], alpha_o[cmp & ~sampled[:, None]]
    err = np.abs(g_s - o_s).max() if g_s.size else 0.0
    _say(f"[{tag}] compared {cmp.sum()}/{verified.sum()} verified positions "
         f"({g_s.size} sampled, max |dalpha| {err:.2e}; {g_g.size} greedy)")
    assert cmp.sum() >= 0.8 * verified.sum()
    assert err < PROB_TOL
    np.testing.assert_array_equal(g_g, o_g)
    return cmp


@pytest.mark.parametrize("B,gamma,V,r,wdtype,greedy", [
    (1, 1, 3, 16, "f32", 0),          # three-token vocabulary
    (5, 3, 17, 16, "bf16", 2),        # one tile, greedy mix
    (33, 4, 1003, 32, "bf16", 3),     # ragged batch and vocabulary
    (70, 6, 4099, 64, "f32", 5),      # f32 weights, several chunks
    (40, 2, 2048 * 3 + 5, 128, "bf16", 0),
    (3, 32, 300, 256, "bf16", 2),     # longest block
    (300, 3, 1024, 16, "bf16", 7),    # more listed rows than one workgroup holds
])
def test_acceptance_parity(B, gamma, V, r, wdtype, greedy):
    cfg, rnd, ell = _case(B, gamma, V, r, wdtype, seed=B * 17 + V, greedy_every=greedy,
                          ell=np.full(B, gamma) if B == 1 else None)
    target = rnd.target_packed(ell)
    _say(f"[alpha] B={B} gamma={gamma} V={V} r={r} {wdtype} greedy_every={greedy} ell={ell.tolist()[:8]}")
    dev = to_device(rnd)
    seed, rid = 19, 2
    d = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, rid)
    alpha = _gpu_alpha(dev, target, ell, d)
    torch.cuda.synchronize()
    od = oracle.draft(rnd.U, rnd.W1, rnd.W2, rnd.anchor, rnd.temperature, seed, rid)
    ao = oracle.acceptance(target, ell, rnd.U, rnd.W1, rnd.W2, rnd.anchor, od["x"], rnd.temperature)
    _compare_alpha(np_of(alpha), np_of(d["x"]), od["x"], ao, rnd.temperature, ell, "alpha")


def test_acceptance_offsets_and_bad_requests():
    """Caller-given offsets equal to the packed layout give the computed-offset
    result; a request with ell out of range, offsets that disagree with its
    ell, or rows past the target is all NaN and leaves the others as they
    were."""
    B, gamma, V, r = 24, 4, 2100, 32
    cfg, rnd, ell = _case(B, gamma, V, r, "bf16", seed=5, greedy_every=5)
    target = rnd.target_packed(ell)
    dev = to_device(rnd)
    d = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], 3, 1)
    a_packed = np_of(_gpu_alpha(dev, target, ell, d))
    # caller-given offsets equal to the packed layout
    a_given = np_of(_gpu_alpha(dev, target, ell, d, row_offsets=S.pack_offsets(ell)))
    np.testing.assert_array_equal(np.isnan(a_given), np.isnan(a_packed))
    np.testing.assert_array_equal(a_given[~np.isnan(a_given)], a_packed[~np.isnan(a_packed)])
    # the same rows spread out with gaps of 2 rows in front of every request:
    # off_{b+1} - off_b = 1 + ell_b fails for all but the last request
    off = np.zeros(B + 1, np.int32)
    spread = np.full((target.shape[0] + 2 * B, V), np.nan, np.float32)
    acc, pos = 0, 0
    for b in range(B):
        pos += 2
        off[b] = pos
        n = 1 + ell[b]
        spread[pos: pos + n] = target[acc: acc + n]
        acc += n
        pos += n
    off[B] = pos
    a_gaps = np_of(_gpu_alpha(dev, spread, ell, d, row_offsets=off))
    assert np.all(np.isnan(a_gaps[:-1]))
    np.testing.assert_array_equal(np.isnan(a_gaps[-1]), np.isnan(a_packed[-1]))
    np.testing.assert_array_equal(a_gaps[-1][~np.isnan(a_gaps[-1])], a_packed[-1][~np.isnan(a_packed[-1])])
    bad = ell.copy()
    bad[3] = gamma + 1
    bad[9] = -1
    a_bad = np_of(_gpu_alpha(dev, target, bad, d))
    assert np.all(np.isnan(a_bad[3])) and np.all(np.isnan(a_bad[9]))
    # the computed layout shifts after a bad ell (it is clamped into range), so
    # compare requests before the first bad one
    np.testing.assert_array_equal(a_bad[:3], a_packed[:3])
    # a short target: the requests whose rows run past it are all NaN
    short = target[: target.shape[0] // 2]
    a_short = np_of(_gpu_alpha(dev, short, ell, d))
    fits = S.pack_offsets(ell)[1:] <= short.shape[0]
    for b in range(B):
        if fits[b]:
            np.testing.assert_array_equal(np.isnan(a_short[b]), np.isnan(a_packed[b]))
        else:
            assert np.all(np.isnan(a_short[b]))


def test_acceptance_large_batch_config():
    """Batch 256, gamma 5, V 129,280, r 256, every position verified: alpha
    against the oracle on every request, and at every sampled
    rejection of the GPU's own verify alpha_j = 1 - S (the residual mass the
    draw kernels sum, an independent reduction)."""
    cfg = S.CONFIGS["large"]
    rnd = S.make_round(cfg)
    ell = np.full(cfg.B, cfg.gamma, np.int32)
    target = rnd.target_packed(ell)
    _say(f"[alpha-large] B={cfg.B} V={cfg.V}")
    dev = to_device(rnd)
    d = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], cfg.seed, 0,
                               margin=True)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    v = gpu_verify(dev, td, ed, d, cfg.seed, 0)
    alpha = np_of(ds.dspark_acceptance(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"],
                                       dev["temperature"]))
    torch.cuda.synchronize()
    assert not np.any(np.isnan(alpha))
    assert np.all((alpha >= 0) & (alpha <= 1 + 1e-5))
    n, resid = np_of(v["n"]), np_of(v["resid"])
    rej = np.nonzero((n < cfg.gamma) & (rnd.temperature > 0))[0]
    assert len(rej) > 100
    err = np.abs(alpha[rej, n[rej]] - (1.0 - resid[rej])).max()
    _say(f"[alpha-large] {len(rej)} sampled rejections: max |alpha_j - (1 - S)| {err:.2e}; "
         f"mean alpha {alpha[rnd.temperature > 0].mean():.3f}")
    assert err < PROB_TOL
    greedy = rnd.temperature == 0
    gx = np_of(d["x"])
    for b in np.nonzero(greedy)[0]:
        assert np.all(alpha[b, :n[b]] == 1.0)
        if n[b] < cfg.gamma:
            assert alpha[b, n[b]] == 0.0
    rows = np.arange(cfg.B)  # every tenth request is greedy
    sub = packed_subset(target, ell, rows)
    od, _ = oracle_round(rnd, sub, ell, cfg.seed, 0, rows=rows)
    ao = oracle.acceptance(sub, ell[rows], rnd.U[rows], rnd.W1, rnd.W2, rnd.anchor[rows], od["x"],
                           rnd.temperature[rows])
    _compare_alpha(alpha[rows], gx[rows], od["x"], ao, rnd.temperature[rows], ell[rows], "alpha-large")
