"""GPU parity: the HIP library against the fp64 oracle on the same seeded
inputs and the same Philox streams, through the C ABI.

Token indices and accepted lengths must be identical for every request whose
decisions all clear their margins (draft and resample Gumbel top-two gaps
> 1e-3, accept tests |u - p/q| > 1e-4; greedy decisions need a top-two logit
gap > 1e-3); probabilities agree within 1e-4.  The rest are counted and
reported.
"""
import dataclasses
import math
import os

import numpy as np
import pytest

import oracle
import synth_inputs as S
from roundkit import (compare_draft, compare_verify, gpu_draft, gpu_verify, np_of, oracle_round, packed_subset,
                      to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import draft_sampling_verification_02_amd as ds  # noqa: E402


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- random streams

@pytest.mark.parametrize("seed", [0, 1, 0xDEADBEEFCAFEF00D])
def test_device_philox_words_match_oracle(seed):
    for stream, k, req, v0, n in [(0, 1, 0, 0, 4096), (0, 5, 255, 129000, 280), (0, 16, 63, 7, 93),
                                  (1, 3, 17, 0, 1), (2, 6, 1023, 0, 300), (3, 2, 9, 0, 4040),
                                  (4, 6, 200, 100, 77)]:
        got = np_of(ds.dspark_debug_random_words(seed, 12345, stream, k, req, v0, n)).view(np.uint32)
        want = np.array([oracle.random_word(seed, 12345, stream, k, req, v0 + i) for i in range(n)], np.uint32)
        np.testing.assert_array_equal(got, want)


def test_device_gumbel_transform_accuracy():
    # every uniform grid point near both ends, and a random sample between
    w = np.concatenate([np.arange(0, 1 << 14, dtype=np.uint64) << 8,
                        (np.uint64(0xFFFFFFFF) - (np.arange(0, 1 << 14, dtype=np.uint64) << 8)),
                        np.random.default_rng(0).integers(0, 2**32, 200000, dtype=np.uint64)]).astype(np.uint32)
    g = np_of(ds.dspark_debug_gumbel(torch.from_numpy(w.view(np.int32)).cuda())).astype(np.float64)
    u = ((w >> 8).astype(np.float64) + 0.5) * 2.0 ** -24
    want = -np.log2(-np.log2(u))
    err = np.abs(g - want)
    _say(f"[gumbel] max error {err.max() * math.log(2):.3g} (natural units) at word {w[np.argmax(err)]:#x}")
    # in natural units the score error is ln2 * err; it must stay far below the 1e-3 draft margin
    assert err.max() * math.log(2) < 2e-5, (err.max(), w[np.argmax(err)])


# ---------------------------------------------------------------- full rounds

_CACHE = {}


def _round(name, rows=None):
    if name not in _CACHE:
        cfg = S.CONFIGS[name]
        rnd = S.make_round(cfg)
        ell = np.full(cfg.B, cfg.gamma, np.int32)
        target = rnd.target_packed(ell)
        _CACHE[name] = (rnd, ell, target)
    return _CACHE[name]


def _run_config(name, oracle_rows=None, round_id=0):
    rnd, ell, target = _round(name)
    cfg = rnd.cfg
    _say(f"[{name}] B={cfg.B} gamma={cfg.gamma} V={cfg.V} r={cfg.r} round={round_id}")
    dev = to_device(rnd)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    d = gpu_draft(dev, cfg.seed, round_id)
    v = gpu_verify(dev, td, ed, d, cfg.seed, round_id)
    torch.cuda.synchronize()
    assert ds.dspark_verify_check(v["workspace"]) == 0
    gd = {k: np_of(t) for k, t in d.items() if k != "workspace"}
    gv = {k: np_of(t) for k, t in v.items() if k != "workspace"}
    rows = oracle_rows
    if rows is None:
        od, ov = oracle_round(rnd, target, ell, cfg.seed, round_id)
        temp, ellr = rnd.temperature, ell
    else:
        od, ov = oracle_round(rnd, packed_subset(target, ell, rows), ell, cfg.seed, round_id, rows=rows)
        temp, ellr = rnd.temperature[rows], ell[rows]
    cd = compare_draft(gd, od, rows=rows)
    _say(f"[{name}] draft:  {cd.report()}")
    cv = compare_verify(gv, od, ov, temp, ellr, rows=rows)
    _say(f"[{name}] verify: {cv.report()}")
    # structural checks on every request
    n, tok, off = gv["n"], gv["tokens"], gv["offsets"]
    assert np.all((n >= 0) & (n <= ell))
    for b in range(cfg.B):
        assert np.all(tok[b, :n[b]] == gd["x"][b, :n[b]])
        assert 0 <= tok[b, n[b]] < cfg.V
        assert np.all(tok[b, n[b] + 1:] == -1)
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(n + 1)]))
    return cd, cv, gd, gv


def test_tiny_config_parity():
    for rid in (0, 1, 2):
        _run_config("tiny", round_id=rid)


def test_tiny_config_many_rounds():
    """Tiny over many rounds: every eligible round matches the oracle."""
    rnd, ell, target = _round("tiny")
    cfg = rnd.cfg
    dev = to_device(rnd)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    mism = inel = 0
    rounds = 300
    for rid in range(rounds):
        d = gpu_draft(dev, cfg.seed, rid)
        v = gpu_verify(dev, td, ed, d, cfg.seed, rid)
        od, ov = oracle_round(rnd, target, ell, cfg.seed, rid)
        gd = {k: np_of(t) for k, t in d.items() if k != "workspace"}
        gv = {k: np_of(t) for k, t in v.items() if k != "workspace"}
        compare_draft(gd, od)
        cv = compare_verify(gv, od, ov, rnd.temperature, ell)
        inel += int((~cv.eligible).sum())
        mism += int(cv.mismatch[~cv.eligible].sum())
    _say(f"[tiny x{rounds}] ineligible rounds={inel} mismatching among them={mism}")
    assert inel <= rounds * 0.05


def test_dspark5_config_parity():
    cd, cv, *_ = _run_config("dspark5")
    assert cd.ineligible_rate < 0.2


def test_large_batch_config_parity():
    cd, cv, gd, gv = _run_config("large")
    assert cd.ineligible_rate < 0.2
    # greedy requests (r % 10 == 0) have q one-hot
    rnd, *_ = _round("large")
    greedy = rnd.temperature == 0
    assert np.all(gd["qx"][greedy] == 1.0)


def test_long_block_config_parity():
    cd, cv, *_ = _run_config("long")
    assert cd.ineligible_rate < 0.3


def test_scheduled_config_parity():
    """Batch 1024: the scheduler's literal choice is ell = 0 everywhere, so
    the GPU verifies 1024 bonus rows; a supplement schedules 256 groups of 4
    requests independently (ell over 0..5).  The oracle checks every request
    of both (one oracle draft, two verifies)."""
    cfg = S.CONFIGS["sched"]
    rnd = S.make_round(cfg)
    sps = S.sps_table_toy(0.2, cfg.B * (1 + cfg.gamma) + 1)
    ell, *_ = ds.dspark_schedule(rnd.c, sps)
    assert np.all(ell == 0)
    # supplement: 256 groups of 4 requests scheduled independently
    ell_g = np.concatenate([ds.dspark_schedule(rnd.c[4 * g:4 * g + 4], S.sps_table_toy(0.2, 25))[0]
                            for g in range(cfg.B // 4)]).astype(np.int32)
    assert len(set(ell_g.tolist())) > 3
    dev = to_device(rnd)
    req = np.asarray(rnd.requests, np.int32)
    od = oracle.draft(rnd.U, rnd.W1, rnd.W2, rnd.anchor, rnd.temperature, cfg.seed, 0, req_ids=req)
    d = gpu_draft(dev, cfg.seed, 0)
    gd = {k: np_of(t) for k, t in d.items() if k != "workspace"}
    cd = compare_draft(gd, od)
    _say(f"[sched] draft {cd.report()}")
    for tag, e in (("literal", ell.astype(np.int32)), ("groups-of-4", ell_g)):
        target = rnd.target_packed(e)
        _say(f"[sched {tag}] rows={target.shape[0]}")
        td = torch.from_numpy(target).cuda()
        ed = torch.from_numpy(e).cuda()
        v = gpu_verify(dev, td, ed, d, cfg.seed, 0)
        torch.cuda.synchronize()
        assert ds.dspark_verify_check(v["workspace"]) == 0
        gv = {k: np_of(t) for k, t in v.items() if k != "workspace"}
        ov = oracle.verify(target, e, rnd.U, rnd.W1, rnd.W2, rnd.anchor, od["x"], rnd.temperature, cfg.seed, 0,
                           req_ids=req)
        cv = compare_verify(gv, od, ov, rnd.temperature, e)
        _say(f"[sched {tag}] verify {cv.report()}")
        n, tok = gv["n"], gv["tokens"]
        assert np.all((n >= 0) & (n <= e))
        for b in range(cfg.B):
            assert np.all(tok[b, :n[b]] == gd["x"][b, :n[b]])
            assert 0 <= tok[b, n[b]] < cfg.V
            assert np.all(tok[b, n[b] + 1:] == -1)
        np.testing.assert_array_equal(gv["offsets"], np.concatenate([[0], np.cumsum(n + 1)]))
        assert cv.ineligible_rate < 0.2


# ---------------------------------------------------------------- edge cases

def _custom_round(B, gamma, V, r, wdtype, seed, greedy_every=0, ell=None, neg_inf_frac=0.0, u_std=3.0,
                  w_std=0.05):
    cfg = S.Config("custom", B=B, gamma=gamma, V=V, r=r, wdtype=wdtype, w_std=w_std, u_std=u_std,
                   noise_std=1.0, seed=seed, greedy_every=greedy_every)
    rnd = S.make_round(cfg)
    if neg_inf_frac > 0:
        mask = np.random.default_rng(seed + 99).uniform(size=rnd.U.shape) < neg_inf_frac
        rnd.U[mask] = -np.inf
    if ell is None:
        ell = np.random.default_rng(seed + 7).integers(0, gamma + 1, B).astype(np.int32)
    target = rnd.target_packed(ell)
    if neg_inf_frac > 0:
        mask = np.random.default_rng(seed + 98).uniform(size=target.shape) < neg_inf_frac
        target[mask] = -np.inf
    return rnd, np.asarray(ell, np.int32), target


@pytest.mark.parametrize("B,gamma,V,r,wdtype,greedy", [
    (1, 1, 3, 16, "f32", 0),          # three-token vocabulary, one position
    (5, 3, 17, 16, "bf16", 0),        # vocabulary inside one tile
    (33, 4, 1003, 32, "bf16", 3),     # ragged batch and vocabulary, greedy mix
    (70, 6, 4099, 64, "f32", 5),      # f32 weights, several tiles and chunks
    (40, 2, 2048 * 3 + 5, 128, "bf16", 0),
    (3, 32, 300, 256, "bf16", 2),     # longest block
    (230, 6, 12288, 64, "bf16", 4),   # a walked batch: rows from the fourth on in the tail kernel
    (320, 4, 8192, 64, "bf16", 5),    # the largest batch with a tail kernel, at the shortest block it serves
    (321, 4, 8192, 64, "bf16", 5),    # one request more: the walk alone
    (200, 9, 4096, 32, "f32", 3),     # f32 weights, a tail of up to seven rows a request
    (200, 5, 4099, 32, "bf16", 4),    # a walked batch whose rows are not 16-byte aligned: scalar loads, no tail
])
def test_edge_shapes_parity(B, gamma, V, r, wdtype, greedy):
    rnd, ell, target = _custom_round(B, gamma, V, r, wdtype, seed=B * 31 + V, greedy_every=greedy)
    _say(f"[edge] B={B} gamma={gamma} V={V} r={r} {wdtype} greedy_every={greedy} ell={ell.tolist()[:8]}")
    dev = to_device(rnd)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    d = gpu_draft(dev, 77, 3)
    v = gpu_verify(dev, td, ed, d, 77, 3)
    assert ds.dspark_verify_check(v["workspace"]) == 0
    gd = {k: np_of(t) for k, t in d.items() if k != "workspace"}
    gv = {k: np_of(t) for k, t in v.items() if k != "workspace"}
    od, ov = oracle_round(rnd, target, ell, 77, 3)
    cd = compare_draft(gd, od)
    cv = compare_verify(gv, od, ov, rnd.temperature, ell)
    _say(f"[edge] draft {cd.report()} | verify {cv.report()}")
    assert cv.eligible.sum() >= 0.5 * B


@pytest.mark.parametrize("B,gamma,V,greedy", [
    (256, 5, 4096, 4),   # walked, rows from the fourth on in the tail kernel
    (600, 3, 4096, 5),   # walked, input checks in a workgroup of their own
    (40, 4, 4096, 3),    # position passes, the last rows in the tail kernel
    (24, 3, 4099, 0),    # position passes, rows not 16-byte aligned
])
def test_drafts_from_the_target_distribution_end_on_the_bonus_token(B, gamma, V, greedy):
    """Zero bias factors make q_k the target's p_k ("DeepSeek DSpark
    explained", section 05: p/q = 1), so every draft passes and every request
    ends with the bonus token from row ell + 1: drawn from p for a sampled
    request (a row the draw reads but the verify passes never need), the row's
    argmax for a greedy one.  Verify lengths are ragged, zero included."""
    rnd, ell, _ = _custom_round(B, gamma, V, 32, "bf16", seed=B + V, greedy_every=greedy)
    rnd = dataclasses.replace(rnd, W1_bits=np.zeros_like(rnd.W1_bits), W2_bits=np.zeros_like(rnd.W2_bits),
                              W1=np.zeros_like(rnd.W1), W2=np.zeros_like(rnd.W2))
    rows = []
    for i in range(B):
        rows.extend(rnd.U[i, k] for k in range(int(ell[i])))
        rows.append(rnd.target_row(i, int(ell[i]) + 1))
    target = np.ascontiguousarray(np.stack(rows), dtype=np.float32)
    _say(f"[bonus] B={B} gamma={gamma} V={V} greedy_every={greedy} ell={ell.tolist()[:8]}")
    dev = to_device(rnd)
    d = gpu_draft(dev, 11, 2)
    v = gpu_verify(dev, torch.from_numpy(target).cuda(), torch.from_numpy(ell).cuda(), d, 11, 2)
    assert ds.dspark_verify_check(v["workspace"]) == 0
    gd = {k: np_of(t) for k, t in d.items() if k != "workspace"}
    gv = {k: np_of(t) for k, t in v.items() if k != "workspace"}
    od, ov = oracle_round(rnd, target, ell, 11, 2)
    np.testing.assert_array_equal(ov["n"], ell)  # the oracle accepts every draft
    cd = compare_draft(gd, od)
    cv = compare_verify(gv, od, ov, rnd.temperature, ell)
    _say(f"[bonus] draft {cd.report()} | verify {cv.report()}")
    assert cv.eligible.sum() >= 0.9 * B
    # an fp32 u q < p can only fail for a uniform within rounding of 1
    assert (gv["n"] == ell).sum() >= B - 1
    assert np.all(gv["resid"][gv["n"] == ell] == -1.0)


def test_neg_inf_logits_parity():
    rnd, ell, target = _custom_round(40, 4, 777, 16, "bf16", seed=5, neg_inf_frac=0.3)
    dev = to_device(rnd)
    d = gpu_draft(dev, 3, 0)
    v = gpu_verify(dev, torch.from_numpy(target).cuda(), torch.from_numpy(ell).cuda(), d, 3, 0)
    gd = {k: np_of(t) for k, t in d.items() if k != "workspace"}
    gv = {k: np_of(t) for k, t in v.items() if k != "workspace"}
    od, ov = oracle_round(rnd, target, ell, 3, 0)
    compare_draft(gd, od)
    compare_verify(gv, od, ov, rnd.temperature, ell)
    # no draft and no emitted token lands on a -inf logit
    for b in range(40):
        for k in range(4):
            assert np.isfinite(rnd.U[b, k, gd["x"][b, k]])


@pytest.mark.parametrize("B,V", [(40, 3001), (256, 3000)])  # position passes / walk and tail kernel
def test_nonfinite_inputs_stay_in_bounds_and_leave_other_requests_alone(B, V):
    """NaN and +inf inputs have no defined result, but a call with them must
    finish, write only where it may, and keep requests independent: base
    logits, target rows and a temperature poisoned for a few requests leave
    every other request's draft, verify and acceptance outputs bit for bit
    as in the clean call, and the poisoned requests still get tokens in
    range, counts within their lengths and -1 padding after them."""
    gamma = 4
    _say(f"[nonfinite] B={B} V={V}")
    rnd, ell, target = _custom_round(B, gamma, V, 64, "bf16", seed=12, greedy_every=6)
    off = S.pack_offsets(ell)

    def run(r, t):
        dev = to_device(r)
        td, ed = torch.from_numpy(t).cuda(), torch.from_numpy(ell).cuda()
        d = gpu_draft(dev, 5, 3)
        v = gpu_verify(dev, td, ed, d, 5, 3)
        a = ds.dspark_acceptance(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"],
                                 dev["temperature"])
        torch.cuda.synchronize()
        assert ds.dspark_verify_check(v["workspace"]) == 0
        out = {k: np_of(x) for k, x in list(d.items()) + list(v.items()) if k != "workspace"}
        out["alpha"] = np_of(a)
        return out

    clean = run(rnd, target)
    bad_u = rnd.U.copy()
    bad_u[3] = np.nan                 # every base logit of a request
    bad_u[7, 1, ::5] = np.nan         # a fifth of one position's
    bad_u[11, 0, 17] = np.inf         # one +inf logit
    bad_u[13, 2] = -np.inf            # a position with no finite logit
    bad_t = target.copy()
    bad_t[off[23]:off[24]] = np.nan   # every target row of a request
    bad_t[off[29] + min(ell[29], 1), 40] = np.inf
    temp = rnd.temperature.copy()
    temp[19] = np.nan
    poisoned = dataclasses.replace(rnd, U=bad_u, temperature=temp)
    got = run(poisoned, bad_t)
    hit = np.zeros(B, bool)
    hit[[3, 7, 11, 13, 19, 23, 29]] = True
    _say(f"[nonfinite] poisoned requests {np.flatnonzero(hit).tolist()}")
    for k in clean:
        if k == "offsets":  # a scan over every request: checked against the counts below
            continue
        a, b = clean[k][~hit], got[k][~hit]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{k} changed for an untouched request"
    np.testing.assert_array_equal(got["offsets"], np.concatenate([[0], np.cumsum(got["n"] + 1)]))
    assert np.all((got["x"] >= 0) & (got["x"] < V))
    n, tok = got["n"], got["tokens"]
    assert np.all((n >= 0) & (n <= ell))
    for b in range(B):
        assert np.all((tok[b, :n[b] + 1] >= 0) & (tok[b, :n[b] + 1] < V)), b
        assert np.all(tok[b, n[b] + 1:] == -1), b


@pytest.mark.parametrize("B,V", [(40, 3001), (256, 3000)])  # position passes / walk and tail kernel
def test_round_replays_from_a_graph_as_it_runs_eagerly(B, V):
    """A round (draft + verify) makes no allocation, memset or host
    synchronisation, so a caller can capture it in a graph: replays, with
    eager rounds of other inputs between them, give the eager outputs bit
    for bit.  Two input sets, each captured once, replayed three times."""
    _say(f"[graph] B={B} V={V}")
    rnd, ell, target = _custom_round(B, 4, V, 64, "bf16", seed=21, greedy_every=5)
    dev = to_device(rnd)
    U2 = (dev["U"] + 0.25).contiguous()
    tds = [torch.from_numpy(target).cuda(), torch.from_numpy(target).cuda() * 0.5]
    ed = torch.from_numpy(ell).cuda()
    d = gpu_draft(dev, 7, 1)
    v = gpu_verify(dev, tds[0], ed, d, 7, 1)

    def step(i):
        U = dev["U"] if i == 0 else U2
        ds.dspark_draft_sample(U, dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], 7, 1 + i, out=d)
        ds.dspark_verify(tds[i], ed, U, dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"], d["qx"],
                         dev["temperature"], 7, 1 + i, out=v)

    keys = ("x", "lse", "qx")
    ref = []
    for i in range(2):
        step(i)
        torch.cuda.synchronize()
        ref.append({k: d[k].clone() for k in keys} | {k: v[k].clone() for k in ("n", "tokens", "offsets")})
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
        step(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for rep in range(3):
        for i in range(2):
            graphs[i].replay()
            torch.cuda.synchronize()
            got = {k: d[k] for k in keys} | {k: v[k] for k in ("n", "tokens", "offsets")}
            for k, t in got.items():
                assert torch.equal(t.view(torch.int32), ref[i][k].view(torch.int32)), (rep, i, k)
            step(1 - i)  # an eager round of the other inputs between replays
            torch.cuda.synchronize()


@pytest.mark.parametrize("B,gamma", [
    (24, 3),   # input checks in the first pass
    (40, 4),   # the same, the block's last rows in the tail kernel
    (600, 3),  # input checks in a prep workgroup, then the walk
    (256, 5),  # input checks in the walk, rows from the fourth on in the tail kernel
])
def test_row_offsets_given_equal_computed_and_bad_ell_flagged(B, gamma):
    rnd, ell, target = _custom_round(B, gamma, 500, 16, "bf16", seed=9)
    _say(f"[offsets] B={B} gamma={gamma}")
    dev = to_device(rnd)
    td = torch.from_numpy(target).cuda()
    d = gpu_draft(dev, 1, 1)
    v1 = gpu_verify(dev, td, torch.from_numpy(ell).cuda(), d, 1, 1)
    off = torch.from_numpy(S.pack_offsets(ell)).cuda()
    v2 = gpu_verify(dev, td, torch.from_numpy(ell).cuda(), d, 1, 1, row_offsets=off)
    assert torch.equal(v1["tokens"], v2["tokens"]) and torch.equal(v1["n"], v2["n"])
    bad = ell.copy()
    bad[5] = 9  # beyond gamma: that request is not verified, the others are
    v3 = gpu_verify(dev, td, torch.from_numpy(bad).cuda(), d, 1, 1)
    assert ds.dspark_verify_check(v3["workspace"]) == ds.DSPARK_ERR_DEVICE_INPUT
    assert int(v3["n"][5]) == -1
    assert np.all(np_of(v3["tokens"][5]) == -1)
    # a packed target two rows short: the last request's rows are out of range
    short = td[:-2].contiguous()
    v4 = gpu_verify(dev, short, torch.from_numpy(ell).cuda(), d, 1, 1)
    assert ds.dspark_verify_check(v4["workspace"]) == ds.DSPARK_ERR_DEVICE_INPUT
    fits = S.pack_offsets(ell)[1:] <= target.shape[0] - 2  # requests whose rows are all there
    assert not fits[-1]
    n4, t4 = np_of(v4["n"]), np_of(v4["tokens"])
    assert np.all(n4[~fits] == -1) and np.all(t4[~fits] == -1)
    np.testing.assert_array_equal(n4[fits], np_of(v1["n"])[fits])
    # and a clean call after the flagged ones reports no error again
    v5 = gpu_verify(dev, td, torch.from_numpy(ell).cuda(), d, 1, 1)
    assert ds.dspark_verify_check(v5["workspace"]) == 0
    assert torch.equal(v5["tokens"], v1["tokens"])


def test_walk_tail_matches_the_walk_alone():
    """A walked request's later rows read by the tail kernel give what the
    walk gives reading them itself.  The first 256 requests of a 600-request
    batch (walked without the tail kernel), verified as a batch of their own
    (rows from the fourth on read by the tail kernel), get the same counts,
    tokens and diagnostics bit for bit, and residual masses within float
    rounding (the draw's chunks follow the batch size).  Random lengths and
    a greedy request in four put requests at every stage of the tail."""
    B, Bs, gamma, V = 600, 256, 6, 8192
    cfg = S.Config("tail", B=B, gamma=gamma, V=V, r=64, wdtype="bf16", w_std=0.05, u_std=3.0, noise_std=0.4,
                   seed=17, greedy_every=4)
    rnd = S.make_round(cfg)
    ell = np.random.default_rng(18).integers(0, gamma + 1, B).astype(np.int32)
    target = rnd.target_packed(ell)
    _say(f"[tail] B={B} / {Bs} gamma={gamma} V={V}")
    dev = to_device(rnd)
    td, ed = torch.from_numpy(target).cuda(), torch.from_numpy(ell).cuda()
    d = gpu_draft(dev, 3, 5)
    full = gpu_verify(dev, td, ed, d, 3, 5)
    sub = {k: (t[:Bs].contiguous() if k in ("U", "anchor", "temperature") else t) for k, t in dev.items()}
    dsub = {k: d[k][:Bs].contiguous() for k in ("x", "lse", "qx")}
    nrows = int(S.pack_offsets(ell)[Bs])
    part = gpu_verify(sub, td[:nrows].contiguous(), ed[:Bs].contiguous(), dsub, 3, 5)
    torch.cuda.synchronize()
    assert ds.dspark_verify_check(full["workspace"]) == 0 and ds.dspark_verify_check(part["workspace"]) == 0
    n_full, n_part = np_of(full["n"])[:Bs], np_of(part["n"])
    reach = [int(np.sum(n_part >= k)) for k in range(3, gamma + 1)]
    _say(f"[tail] requests with at least 3 .. {gamma} drafts accepted: {reach}")
    assert reach[0] >= 40 and reach[-1] >= 5
    np.testing.assert_array_equal(n_part, n_full)
    np.testing.assert_array_equal(np_of(part["tokens"]), np_of(full["tokens"])[:Bs])
    assert np.array_equal(np_of(part["diag"]).view(np.uint32), np_of(full["diag"])[:Bs].view(np.uint32))
    np.testing.assert_allclose(np_of(part["resid"]), np_of(full["resid"])[:Bs], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("B,gamma,V,kernels", [
    (256, 5, 4096, {"verify_walk", "verify_tail"}),  # a walked batch with a tail
    (320, 4, 4096, {"verify_walk", "verify_tail"}),  # the largest such batch, the shortest such block
    (321, 5, 4096, {"verify_walk"}),                 # one request more
    (256, 3, 4096, {"verify_walk"}),                 # a block too short for a tail
    (256, 5, 4099, {"verify_walk"}),                 # rows that take scalar loads
    (191, 5, 4096, {"verify_pass1"}),                # below the walk: position passes (too many rows for the tail)
    (40, 4, 4096, {"verify_pass1", "verify_tail"}),  # small rows: the passes hand the last four to the tail kernel
    (40, 4, 4099, {"verify_pass1"}),                 # the same with rows that take scalar loads: passes only
    (24, 1, 4096, {"verify_pass1"}),                 # one draft: both rows in the first pass
])
def test_verify_launches_the_kernels_its_shape_calls_for(B, gamma, V, kernels):
    """Which verify kernels a call launches, read back from the library's
    launch profiler: the walk from 192 requests on, with the tail kernel up to
    320 requests, blocks of at least 4 drafts and 16-byte aligned rows; below
    192 the position passes, which hand the block's last rows to the tail
    kernel when that saves launches and the rows it may read are few and
    cheap."""
    rnd, ell, target = _custom_round(B, gamma, V, 32, "bf16", seed=B + gamma, greedy_every=5)
    _say(f"[launches] B={B} gamma={gamma} V={V}")
    dev = to_device(rnd)
    td, ed = torch.from_numpy(target).cuda(), torch.from_numpy(ell).cuda()
    d = gpu_draft(dev, 1, 2)
    torch.cuda.synchronize()
    ds.dspark_profile_reset()
    ds.dspark_profile_enable(True)
    try:
        v = gpu_verify(dev, td, ed, d, 1, 2)
        torch.cuda.synchronize()
        ds.dspark_profile_collect()
    finally:
        ds.dspark_profile_enable(False)
    launched = {k for k, (n, _) in ds.dspark_profile_read().items() if n > 0 and k.startswith("verify_")}
    ds.dspark_profile_reset()
    assert ds.dspark_verify_check(v["workspace"]) == 0
    for k in ("verify_walk", "verify_tail", "verify_pass1"):
        assert (k in launched) == (k in kernels), (k, sorted(launched))
    assert {"verify_draw", "verify_finish"} <= launched


@pytest.mark.parametrize("name", ["dspark5", "large"])  # position passes / walk and tail kernel
def test_bitwise_determinism(name):
    _say(f"[determinism] {name}")
    rnd, ell, target = _round(name)
    dev = to_device(rnd)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    outs = []
    for _ in range(2):
        d = gpu_draft(dev, 1, 42)
        v = gpu_verify(dev, td, ed, d, 1, 42)
        outs.append({k: t.clone() for k, t in list(d.items()) + [("n", v["n"]), ("tokens", v["tokens"]),
                                                                  ("diag", v["diag"]), ("resid", v["resid"])]
                     if k != "workspace"})
    for k in outs[0]:
        a, b = outs[0][k], outs[1][k]
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), k


# ---------------------------------------------------------------- statistics

def test_worked_example_section05_on_gpu():
    """q = (0.70, 0.18, 0.12), p = (0.50, 0.30, 0.20) through the GPU kernels
    (U = ln q, W2 = 0, target = ln p): acceptance 0.80, residual (0, 0.6, 0.4),
    emitted tokens distributed as p (chi-square, 2 dof, 13.82 at alpha 1e-3)."""
    q = np.array([0.70, 0.18, 0.12])
    p = np.array([0.50, 0.30, 0.20])
    B, rounds = 50000, 20
    V, r = 3, 16
    U = torch.from_numpy(np.broadcast_to(np.log(q).astype(np.float32), (B, 1, V)).copy()).cuda()
    W = torch.zeros((V, r), dtype=torch.bfloat16, device="cuda")
    anchor = torch.zeros(B, dtype=torch.int32, device="cuda")
    temp = torch.ones(B, dtype=torch.float32, device="cuda")
    ell = torch.ones(B, dtype=torch.int32, device="cuda")
    target = torch.from_numpy(np.broadcast_to(np.log(p).astype(np.float32), (2 * B, V)).copy()).cuda()
    acc = 0
    counts = np.zeros(3)
    rcounts = np.zeros(3)
    for rid in range(rounds):
        d = ds.dspark_draft_sample(U, W, W, anchor, temp, 2024, rid)
        v = ds.dspark_verify(target, ell, U, W, W, anchor, d["x"], d["lse"], d["qx"], temp, 2024, rid, resid=True)
        n = np_of(v["n"])
        y = np_of(v["tokens"][:, 0])
        acc += int((n == 1).sum())
        counts += np.bincount(y, minlength=3)
        rcounts += np.bincount(y[n == 0], minlength=3)
        res = np_of(v["resid"])[n == 0]
        np.testing.assert_allclose(res, 0.2, atol=1e-5)
    N = B * rounds
    rate = acc / N
    assert abs(rate - 0.8) < 3 * math.sqrt(0.16 / N), rate
    chi2 = (((counts - N * p) ** 2) / (N * p)).sum()
    assert chi2 < 13.82, chi2
    assert rcounts[0] == 0
    rp = np.array([0.6, 0.4])
    chi2r = (((rcounts[1:] - rcounts.sum() * rp) ** 2) / (rcounts.sum() * rp)).sum()
    assert chi2r < 10.83, chi2r
    _say(f"[worked example] acceptance={rate:.5f} chi2(p)={chi2:.2f} chi2(residual)={chi2r:.2f}")


def test_q_equals_p_accepts_all_on_gpu():
    V, r, B, gamma = 5, 16, 4096, 3
    logits = np.log(np.array([0.1, 0.2, 0.3, 0.15, 0.25])).astype(np.float32)
    U = torch.from_numpy(np.broadcast_to(logits, (B, gamma, V)).copy()).cuda()
    W = torch.zeros((V, r), dtype=torch.bfloat16, device="cuda")
    anchor = torch.zeros(B, dtype=torch.int32, device="cuda")
    temp = torch.ones(B, dtype=torch.float32, device="cuda")
    ell = torch.full((B,), gamma, dtype=torch.int32, device="cuda")
    target = torch.from_numpy(np.broadcast_to(logits, (B * (gamma + 1), V)).copy()).cuda()
    full = total = 0
    for rid in range(5):
        d = ds.dspark_draft_sample(U, W, W, anchor, temp, 5, rid)
        v = ds.dspark_verify(target, ell, U, W, W, anchor, d["x"], d["lse"], d["qx"], temp, 5, rid)
        full += int((v["n"] == gamma).sum())
        total += B
    # p/q = 1 up to float32 rounding: only a uniform within ~1e-7 of 1 can fail
    assert total - full <= 2, (total, full)


# ---------------------------------------------------------------- bias product alone

@pytest.mark.parametrize("B,V,r,wdtype", [
    (70, 4099, 64, "f32"),             # ragged batch and vocabulary, several chunks
    (256, 2048 * 3 + 5, 256, "bf16"),  # headline rank, ragged tail tile
    (33, 17, 16, "bf16"),              # vocabulary inside one tile
    (64, 40000, 128, "bf16"),          # chunks of three two-tile stages
    (100, 50007, 32, "bf16"),          # four stages a chunk; half the waves stage the W2 rows
    (256, 98309, 256, "bf16"),         # seven stages a chunk, a shorter last chunk with a tail
    (64, 40000, 128, "f32"),           # f32 factors through the same stage ring
    (256, 129280, 256, "bf16"),        # the large-batch round's shape
    (270, 9001, 256, "bf16"),          # nine request blocks: a second workgroup with one block
])
def test_bias_gemm_rowmax_matches_fp64(B, V, r, wdtype):
    """The matrix-unit tiling of the draft step on its own: rowmax[b] =
    max_v W1[idx_b] . W2[v] against the same sums in fp64 (on a sample of rows
    at the larger shapes).  The products of exact bf16 / f32 values are summed
    in fp32, so each sum is within r * 2^-24 * sum |terms| of the fp64 one
    (the classic bound, doubled)."""
    rnd, _, _ = _custom_round(B, 1, V, r, wdtype, seed=B + V + r)
    dev = to_device(rnd)
    idx = np.random.default_rng(V).integers(0, V, B).astype(np.int32)
    _say(f"[bias_gemm] B={B} V={V} r={r} {wdtype}")
    out = ds.dspark_debug_bias_gemm(dev["W1"], dev["W2"], torch.from_numpy(idx).cuda())
    got = np_of(out["rowmax"])
    rows = np.arange(B) if B * V <= 4_000_000 else np.random.default_rng(B).choice(B, 24, replace=False)
    w1 = rnd.W1[idx[rows]].astype(np.float64)
    w2t = rnd.W2.astype(np.float64).T
    ref = (w1 @ w2t).max(axis=1)
    scale = np.abs(w1) @ np.abs(w2t)
    tol = 2 * r * 2.0 ** -24 * scale.max(axis=1) + 1e-7
    err = np.abs(got[rows] - ref)
    assert np.all(err <= tol), (np.max(err / tol), rows[np.argmax(err / tol)])
