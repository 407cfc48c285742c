"""Shared pieces of the GPU parity tests: move a synthetic round to the
device, run the library's draft + verify, run the oracle on the same inputs,
and split requests into those whose every decision clears its margin
(compared exactly) and the rest (counted)."""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import synth_inputs as S

DRAFT_MARGIN = 1e-3  # Gumbel top-two score gap below which a draft pick may flip
ACCEPT_MARGIN = 1e-4  # |u - p/q| below which an accept test may flip
PICK_MARGIN = 1e-3  # Gumbel top-two score gap of the resample / bonus draw
GREEDY_MARGIN = 1e-3  # top-two target logit gap for greedy decisions
PROB_TOL = 1e-4  # absolute tolerance on probabilities


def to_device(rnd: S.Round, device="cuda"):
    import torch
    W1h, W2h = rnd.weights_device_layout()
    if rnd.cfg.wdtype == "bf16":
        W1 = torch.from_numpy(W1h.view(np.int16)).to(device).view(torch.bfloat16)
        W2 = torch.from_numpy(W2h.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        W1 = torch.from_numpy(W1h).to(device)
        W2 = torch.from_numpy(W2h).to(device)
    return {
        "U": torch.from_numpy(rnd.U).to(device),
        "W1": W1,
        "W2": W2,
        "anchor": torch.from_numpy(rnd.anchor).to(device),
        "temperature": torch.from_numpy(rnd.temperature).to(device),
    }


def gpu_draft(dev, seed, round_id, margin=True):
    import draft_sampling_verification_02_amd as ds
    out = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"],
                                 seed, round_id, margin=margin)
    return out


def gpu_verify(dev, target_dev, ell_dev, d, seed, round_id, row_offsets=None):
    import draft_sampling_verification_02_amd as ds
    return ds.dspark_verify(target_dev, ell_dev, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"],
                            d["qx"], dev["temperature"], seed, round_id, row_offsets=row_offsets,
                            diag=True, resid=True)


def np_of(t):
    return t.detach().cpu().numpy()


@dataclasses.dataclass
class Compare:
    n_req: int
    eligible: np.ndarray  # bool [B]
    mismatch: np.ndarray  # bool [B]

    @property
    def ineligible_rate(self):
        return float((~self.eligible).mean()) if self.n_req else 0.0

    def report(self):
        inel = ~self.eligible
        mis_inel = float(self.mismatch[inel].mean()) if inel.any() else 0.0
        return (f"requests={self.n_req} ineligible={inel.sum()} ({self.ineligible_rate:.3%}) "
                f"mismatch(eligible)={int(self.mismatch[self.eligible].sum())} "
                f"mismatch rate among ineligible={mis_inel:.2f}")


def draft_eligible(orc_draft):
    return np.all(orc_draft["margin"] > DRAFT_MARGIN, axis=1)


def compare_draft(gd, od, rows=None, strict=True):
    """gd: GPU draft outputs (numpy dict), od: oracle draft outputs.  strict
    asserts on eligible requests; otherwise only counts."""
    x, lse, qx = gd["x"], gd["lse"], gd["qx"]
    if rows is not None:
        x, lse, qx = x[rows], lse[rows], qx[rows]
    el = draft_eligible(od)
    mism = np.any(x != od["x"], axis=1)
    # probabilities on eligible requests
    if strict and el.any():
        np.testing.assert_array_equal(x[el], od["x"][el])
        np.testing.assert_allclose(qx[el], od["qx"][el], rtol=0, atol=PROB_TOL)
        # lse is a log; compare as the probability scale it sets: |dlse| small
        np.testing.assert_allclose(lse[el], od["lse"][el], rtol=0, atol=1e-3)
        np.testing.assert_allclose(np.exp(od["lse"][el] - lse[el]), 1.0, rtol=0, atol=PROB_TOL)
    return Compare(len(el), el, mism)


def verify_eligible(od, ov, temperature, ell):
    el = draft_eligible(od)
    B = len(el)
    for b in range(B):
        if not el[b]:
            continue
        n = ov["n"][b]
        L = ell[b]
        tested = min(n + 1, L)
        am = ov["accept_margin"][b, :tested]
        thr = ACCEPT_MARGIN if temperature[b] > 0 else GREEDY_MARGIN
        if np.any(am <= thr):
            el[b] = False
            continue
        pthr = PICK_MARGIN if temperature[b] > 0 else GREEDY_MARGIN
        if not ov["pick_margin"][b] > pthr:
            el[b] = False
    return el


def compare_verify(gv, od, ov, temperature, ell, rows=None, strict=True):
    n, tokens, diag, resid = gv["n"], gv["tokens"], gv["diag"], gv["resid"]
    if rows is not None:
        n, tokens, diag, resid = n[rows], tokens[rows], diag[rows], resid[rows]
    el = verify_eligible(od, ov, temperature, ell)
    mism = (n != ov["n"]) | np.any(tokens != ov["tokens"], axis=1)
    if strict and el.any():
        np.testing.assert_array_equal(n[el], ov["n"][el])
        np.testing.assert_array_equal(tokens[el], ov["tokens"][el])
        dg, do = diag[el], ov["diag"][el]
        tested = ~np.isnan(do)
        assert np.array_equal(np.isnan(dg), ~tested)
        np.testing.assert_allclose(dg[tested], do[tested], rtol=0, atol=PROB_TOL)
        np.testing.assert_allclose(resid[el], ov["resid"][el], rtol=0, atol=PROB_TOL)
    return Compare(len(el), el, mism)


def oracle_round(rnd: S.Round, target, ell, seed, round_id, rows=None):
    """Oracle draft + verify on the round's inputs (optionally a subset of
    request rows, with their global request indices)."""
    U, anchor, temp = rnd.U, rnd.anchor, rnd.temperature
    req = np.asarray(rnd.requests, np.int32)
    if rows is not None:
        U, anchor, temp, req = U[rows], anchor[rows], temp[rows], req[rows]
    od = oracle.draft(U, rnd.W1, rnd.W2, anchor, temp, seed, round_id, req_ids=req)
    ov = oracle.verify(target, np.asarray(ell)[rows] if rows is not None else ell, U, rnd.W1, rnd.W2, anchor,
                       od["x"], temp, seed, round_id, req_ids=req)
    return od, ov


def packed_subset(target, ell, rows):
    off = S.pack_offsets(ell)
    parts = [target[off[b]:off[b + 1]] for b in rows]
    return np.ascontiguousarray(np.concatenate(parts, axis=0))
