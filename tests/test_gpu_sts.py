"""GPU parity of sequential temperature scaling (page "DSpark：DeepSeek
线上跑的投机解码..." (marsggbo.github.io), section 4.2) and of the calibrated
confidence head, through the C ABI, against the fp64 oracle on the same
seeded inputs.

The GPU bins float32 survival products, the oracle double ones, so a sample
within rounding of a bin edge may land in the neighbouring bin: each such
sample moves an ECE by at most 2/N_k.  ECE curves are compared within 6/N_k;
the chosen temperature is compared exactly at the positions where the
oracle's best grid value beats every other by more than 12/N_k, up to the
first position that does not (later positions build on the choice).
"""
import numpy as np
import pytest

import oracle
import synth_inputs as S
from roundkit import np_of, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import draft_sampling_verification_02_amd as ds  # noqa: E402


def _say(msg):
    print(msg, flush=True)


GRID = np.round(np.arange(0.25, 4.0001, 0.05), 2).astype(np.float32)


def _fit_both(c, n, ell=None, n_bins=15, grid=GRID):
    g = ds.dspark_sts_fit(torch.from_numpy(c).cuda(), torch.from_numpy(n).cuda(), torch.from_numpy(grid).cuda(),
                          ell=None if ell is None else torch.from_numpy(ell).cuda(), n_bins=n_bins, ece_grid=True)
    torch.cuda.synchronize()
    tau_o, ece_o, eg_o = oracle.sts_fit(c, n, grid, n_bins=n_bins, ell=ell)
    return {k: np_of(v) for k, v in g.items()}, tau_o, ece_o, eg_o


def _compare(g, tau_o, ece_o, eg_o, c, ell, tag):
    N, gamma = c.shape
    L = np.full(N, gamma) if ell is None else ell
    same_so_far = True
    for k in range(gamma):
        Nk = int(((L >= k + 1) & (L <= gamma)).sum())
        if Nk == 0:
            assert g["tau"][k] == 1.0 and np.isnan(g["ece"][k]) and np.isnan(ece_o[k])
            continue
        if not same_so_far:
            break
        fin = np.isfinite(eg_o[k])
        err = np.abs(g["ece_grid"][k][fin] - eg_o[k][fin]).max()
        assert err <= 6.0 / Nk + 1e-6, f"{tag} k={k + 1}: ECE curve off by {err:.2e}"
        assert np.all(np.isinf(g["ece_grid"][k][~fin]))
        order = np.sort(eg_o[k][fin])
        gap = order[1] - order[0] if len(order) > 1 else np.inf
        if gap > 12.0 / Nk:
            assert g["tau"][k] == tau_o[k], f"{tag} k={k + 1}: tau {g['tau'][k]} vs {tau_o[k]}"
            assert abs(g["ece"][k] - ece_o[k]) <= 6.0 / Nk + 1e-6
        else:
            same_so_far = g["tau"][k] == tau_o[k]
        _say(f"[{tag}] k={k + 1}: tau {g['tau'][k]:.2f} (oracle {tau_o[k]:.2f}), ECE {g['ece'][k]:.4f} "
             f"(oracle {ece_o[k]:.4f}), best-vs-next gap {gap:.1e}, curve error {err:.1e}, N_k {Nk}")


@pytest.mark.parametrize("N,scales,n_bins", [
    (200_000, [2.0, 0.5, 1.0], 15),
    (50_000, [1.5, 1.5, 0.7, 3.0, 1.0], 10),
    (1_000, [2.0, 1.0], 20),        # fewer samples than one grid step resolves
    (257, [1.0], 15),               # a ragged last workgroup
])
def test_sts_fit_parity(N, scales, n_bins):
    c, n = S.sts_samples(N, scales, seed=N + len(scales))
    g, tau_o, ece_o, eg_o = _fit_both(c, n, n_bins=n_bins)
    _compare(g, tau_o, ece_o, eg_o, c, None, f"sts N={N}")


def test_sts_fit_ragged_verify_lengths_and_edge_grid():
    """Samples that verified fewer positions drop out where they stop; grid
    values <= 0 are never chosen; a position nobody verified keeps tau = 1."""
    c, n = S.sts_samples(30_000, [2.0, 0.5, 1.0, 1.0], seed=5)
    ell = np.random.default_rng(6).integers(0, 4, len(c)).astype(np.int32)  # nobody verifies position 4
    n = np.minimum(n, ell).astype(np.int32)
    grid = np.concatenate([np.float32([-1.0, 0.0]), GRID])
    g, tau_o, ece_o, eg_o = _fit_both(c, n, ell=ell, grid=grid)
    _compare(g, tau_o, ece_o, eg_o, c, ell, "sts ragged")
    assert g["tau"][3] == 1.0 and np.isnan(g["ece"][3])


def test_sts_is_deterministic():
    c, n = S.sts_samples(100_000, [2.0, 0.5], seed=8)
    a, _, _, _ = _fit_both(c, n)
    b, _, _, _ = _fit_both(c, n)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_calibrated_head_parity():
    """The fused head with per-position temperatures against the oracle's
    calibrated head on the same drafts."""
    B, gamma, V, r, d = 64, 5, 3001, 64, 256
    cfg = S.Config("custom", B=B, gamma=gamma, V=V, r=r, wdtype="bf16", w_std=0.05, u_std=3.0, noise_std=1.0,
                   seed=31, greedy_every=4)
    rnd = S.make_round(cfg)
    h, w = S.confidence_head_inputs(cfg, d)
    tau = np.array([0.5, 1.0, 1.7, 2.5, 4.0], np.float32)
    dev = to_device(rnd)
    gc = ds.dspark_draft_sample_confidence(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"],
                                           torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(), 3, 1,
                                           conf_tau=torch.from_numpy(tau).cuda())
    torch.cuda.synchronize()
    od = oracle.draft(rnd.U, rnd.W1, rnd.W2, rnd.anchor, rnd.temperature, 3, 1)
    c, a = oracle.confidence(h, w, rnd.W1, rnd.anchor, od["x"], tau=tau)
    gx = np_of(gc["x"])
    ok = np.ones_like(gx, bool)
    ok[:, 1:] = np.cumprod(gx[:, :-1] == od["x"][:, :-1], axis=1).astype(bool)
    assert ok.mean() > 0.9
    np.testing.assert_allclose(np_of(gc["conf"])[ok], c[ok], rtol=0, atol=1e-4)
    np.testing.assert_allclose(np_of(gc["survival"])[ok], a[ok], rtol=0, atol=1e-4)


def test_sts_on_the_rounds_own_outcomes():
    """Calibration from the library's own rounds: 40 rounds of the fused head
    and the verify kernel (B = 64, V = 20,000), then the fit.  The outcomes
    come from the GPU, so this checks what holds for any input: the chosen
    tau is the first minimum of its ECE curve, and no worse than tau = 1."""
    B, gamma, V, r, d = 64, 5, 20_000, 64, 256
    cfg = S.Config("custom", B=B, gamma=gamma, V=V, r=r, wdtype="bf16", w_std=0.05, u_std=3.0, noise_std=1.0,
                   seed=41, greedy_every=10)
    rnd = S.make_round(cfg)
    h, w = S.confidence_head_inputs(cfg, d)
    ell = np.full(B, gamma, np.int32)
    dev = to_device(rnd)
    td = torch.from_numpy(rnd.target_packed(ell)).cuda()
    ed = torch.from_numpy(ell).cuda()
    hd, wd = torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda()
    cs, ns = [], []
    for rid in range(40):
        gc = ds.dspark_draft_sample_confidence(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"],
                                               hd, wd, 5, rid)
        v = ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], gc["x"], gc["lse"], gc["qx"],
                             dev["temperature"], 5, rid)
        cs.append(gc["conf"].clone())
        ns.append(v["n"].clone())
    conf = torch.cat(cs)
    nacc = torch.cat(ns)
    grid = torch.from_numpy(GRID).cuda()
    fit = ds.dspark_sts_fit(conf, nacc, grid, ece_grid=True)
    torch.cuda.synchronize()
    tau, ece, eg = np_of(fit["tau"]), np_of(fit["ece"]), np_of(fit["ece_grid"])
    one = int(np.argmin(np.abs(GRID - 1.0)))
    for k in range(gamma):
        i = int(np.argmin(eg[k]))  # numpy takes the first minimum
        assert tau[k] == GRID[i] and ece[k] == eg[k, i] and ece[k] <= eg[k, one]
    _say(f"[sts-own] tau {tau.tolist()}, ECE {np.round(ece, 4).tolist()} (tau = 1: {np.round(eg[:, one], 4).tolist()})")
