#!/usr/bin/env python3
"""Benchmark: one DSpark draft-and-verify round per step on one MI355X.

Workload: the large-batch round -- B = 256 requests, gamma = 5 block
positions, V = 129,280 vocabulary, rank r = 256 bf16 Markov factors, float32
base and target logits, 10% greedy requests, every drafted position verified
(ell = gamma).  Inputs are seeded synthetic data already resident in HBM when
the timed region starts.  A step is dspark_draft_sample + dspark_verify over
the whole batch; round_id advances every step.

Order of the run: round 0 on the GPU; the CPU oracle on the same round (the
parity gate and the CPU baseline); the other configurations, each
parity-gated against the oracle on every request and timed with the oracle
beside it; the secondary GPU measurements; the single-round time
distribution; then the W warmup rounds and the K timed rounds; then a second
pass of K rounds with per-kernel HIP events
(and each round's outcome counts, from which the logit passes' bytes are
counted).  The printed JSON line carries the headline throughput (drafted
positions per second), the dominant kernel's roofline figures measured with
HIP events on the launch stream (W2 warm, as in the timed rounds, and cold),
and the CPU oracle timed on this host.

Secondary figures: the distribution of single-round times, every
configuration's round, the bias product alone (the draft step's MFMA tiling
without U_k or sampling) with W2 warm in the last-level cache and after a
512 MiB flush, the draft step with every step's inputs evicted, the host
scheduler on a 1024-request batch, the round with the confidence head, the
acceptance-probability labelling pass, the RNN head's round, the calibration
fit of the head on 200,000 synthetic samples, and the oracle on one thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
KERNEL_SOURCES = ["draft_sampling_verification_02_amd/csrc/draft.hip",
                  "draft_sampling_verification_02_amd/csrc/stage.hpp",
                  "draft_sampling_verification_02_amd/csrc/device_common.hpp"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "draft_step_large_batch_counters.md")
INPUT_COPIES = 3  # copies of U and the target the timed rounds take in turn


def _kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_from_counters(launch_bytes):
    """HBM bytes per draft_step launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    m = re.search(r"kernel source hash:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm bytes per launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != _kernel_hash():
        return None
    return float(t.group(1))


def _logit_passes(phases, outcome, B, V, r):
    """The verify's logit passes against the HBM peak: algorithmic bytes over
    the event-timed average launch, the bytes counted from the outcomes of the
    same timed rounds (averages per round).  The walk reads rows 1 .. n + 1 of
    every request (up to the first rejection's row, or the bonus row of a
    greedy request; a sampled request's bonus row is the draw's alone), timed
    with the tail kernel that reads a batch's last rows when it has one (the
    tail's rows past a rejection are read but not counted); the draw reads the
    target and U_j rows of every residual draw, the target row of every
    bonus draw, and W2 once when any draw is a residual one."""
    row = V * 4
    out = {}

    def put(name, nbytes, keys):
        us = sum(phases.get(k, {}).get("avg_us", 0.0) for k in keys)
        if us > 0:
            gbs = nbytes / (us * 1e-6) / 1e9
            out[name] = {"bytes": int(nbytes), "us": round(us, 2), "gbs": round(gbs, 1),
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}

    if "verify_walk" in phases:  # (the position passes of a small batch may end in the tail kernel too)
        put("verify_walk", outcome["rows"] * row, ("verify_walk", "verify_tail"))
    put("verify_draw", (2 * outcome["residual"] + outcome["bonus"]) * row + (V * r * 2 if outcome["residual"] else 0),
        ("verify_draw",))
    out["per_round"] = {k: round(v, 2) for k, v in outcome.items()}
    return out


def _outcome_counter(torch, temperature, ell):
    """Accumulates, on the device, each round's rows read by the walk
    (sum of n + 1, less the sampled bonus rows, which only the draw reads),
    residual draws (sampled, n < ell) and bonus draws (sampled, n = ell);
    .mean() gives the averages per round."""
    sampled = temperature > 0
    acc = torch.zeros(3, dtype=torch.float64, device=temperature.device)
    cnt = [0]

    def add(n):
        res = ((n < ell) & sampled).sum()
        bon = ((n == ell) & sampled).sum()
        rows = (n + 1).sum() - bon
        acc.add_(torch.stack([rows, res, bon]).to(torch.float64))
        cnt[0] += 1

    def mean():
        a = acc.cpu().numpy() / max(1, cnt[0])
        return {"rows": float(a[0]), "residual": float(a[1]), "bonus": float(a[2])}

    return add, mean


def _round_distribution(torch, step, n, base):
    """Single-round times (HIP events on the launch stream around each round,
    rounds queued back to back): p10 / p50 / p90 in milliseconds."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        step(base + i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"rounds": n, "p10": round(float(np.percentile(t, 10)), 5), "p50": round(float(np.median(t)), 5),
            "p90": round(float(np.percentile(t, 90)), 5)}


class _Evict:
    """Evicts the last-level cache by reading a 512 MiB buffer (a read
    leaves clean lines, so the kernel measured next does not compete with
    the write-back that a flush by writing would leave behind)."""

    def __init__(self, torch):
        self.buf = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.buf.sum()


def _bias_gemm_alone(torch, ds, dev, B, V, r, reps=30):
    """The bias product B = W1[idx] . W2^T of one draft step with the step's
    tiling and a running maximum as its only epilogue.  Warm: launches back to
    back, so W2 (V*r*2 bytes) stays in the last-level cache; cold: a 512 MiB
    read between launches evicts it.  Times are HIP events around the kernel
    alone, on the launch stream."""
    g = torch.Generator(device="cpu").manual_seed(7)
    idx = torch.randint(0, V, (B,), generator=g, dtype=torch.int32).cuda()
    out = ds.dspark_debug_bias_gemm(dev["W1"], dev["W2"], idx)
    evict = _Evict(torch)
    flops = 2.0 * B * r * V
    res = {"flops_per_launch": flops, "w2_bytes": V * r * 2}
    for mode in ("warm", "cold"):
        torch.cuda.synchronize()
        ds.dspark_profile_reset()
        ds.dspark_profile_enable(True)
        for i in range(reps):
            if mode == "cold":
                evict()
            ds.dspark_debug_bias_gemm(dev["W1"], dev["W2"], idx, out=out)
        torch.cuda.synchronize()
        ds.dspark_profile_collect()
        ds.dspark_profile_enable(False)
        n, ms = ds.dspark_profile_read()["bias_gemm"]
        us = 1e3 * ms / n
        tf = flops / (us * 1e-6) / 1e12
        res[mode] = {"avg_us": round(us, 2), "tflops": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "w2_gbs": round(V * r * 2 / (us * 1e-6) / 1e9, 1)}
    return res


def _schedule_time(ds, S, reps=400):
    """Host scheduler on the scheduled-batch workload (1024 requests, gamma 5,
    confidences ~ Beta(8, 2), SPS(B) tabulated for every batch size): median
    and p90 microseconds per call, including the ctypes call; the same for
    the production-style scheduler at a capacity from its history rule."""
    import numpy as np
    cfg = S.CONFIGS["sched"]
    c = np.random.default_rng((cfg.seed, 5)).beta(8.0, 2.0, size=(cfg.B, cfg.gamma))
    sps = S.sps_table_toy(0.5, cfg.B * (1 + cfg.gamma) + 1)
    ds.dspark_schedule(c, sps)
    t = []
    for _ in range(reps):
        t0 = time.perf_counter_ns()
        ds.dspark_schedule(c, sps)
        t.append((time.perf_counter_ns() - t0) / 1e3)
    t = np.array(t)
    # the production-style scheduler at a capacity of half the drafts (its
    # history rule from two previous steps with B/R = 3.5 and 2.5)
    cap = ds.dspark_history_capacity([cfg.B * 7 // 2, cfg.B * 5 // 2], [cfg.B, cfg.B], cfg.B, cfg.gamma)
    tc = []
    for _ in range(reps):
        t0 = time.perf_counter_ns()
        ds.dspark_schedule_capacity(c, cap)
        tc.append((time.perf_counter_ns() - t0) / 1e3)
    tc = np.array(tc)
    return {"requests": cfg.B, "gamma": cfg.gamma, "sps_len": len(sps), "p50_us": round(float(np.median(t)), 2),
            "p90_us": round(float(np.percentile(t, 90)), 2),
            "capacity": {"capacity": cap, "p50_us": round(float(np.median(tc)), 2),
                         "p90_us": round(float(np.percentile(tc, 90)), 2)}}


def _oracle_one_thread(rnd, target, ell, seed, gamma, oracle_round, rows=128):
    """The oracle restricted to one OpenMP thread on the first `rows` requests
    of the same round (a bounded sample of a few seconds)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from roundkit import packed_subset
    sel = np.arange(rows)
    tgt = packed_subset(target, ell, sel)
    with threadpool_limits(limits=1):
        omp = [i for i in threadpool_info() if i.get("user_api") == "openmp"]
        threads = max([i["num_threads"] for i in omp], default=1)
        t0 = time.time()
        oracle_round(rnd, tgt, ell, seed, 0, rows=sel)
        dt = time.time() - t0
    return {"value": round(rows * gamma / dt, 2), "unit": "drafted positions/s", "cores": threads,
            "sample": f"requests 0..{rows - 1} of the same round: fp64 draft + verify, {dt:.1f}s"}


def _profiled(torch, ds, fn, reps):
    """Per-kernel HIP-event averages (microseconds) of `reps` calls of fn."""
    torch.cuda.synchronize()
    ds.dspark_profile_reset()
    ds.dspark_profile_enable(True)
    for i in range(reps):
        fn(i)
    torch.cuda.synchronize()
    ds.dspark_profile_collect()
    ds.dspark_profile_enable(False)
    return {k: 1e3 * ms / max(1, n) for k, (n, ms) in ds.dspark_profile_read().items()}


def _events_ms(torch, fn, reps, base):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(base + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _confidence_head(torch, ds, S, cfg, dev, td, ed, seed, reps):
    """The round with the confidence head fused into the draft (d = 1024,
    synthetic h and w): round time and the draft reduce's time, against the
    plain round measured the same way."""
    h, w = S.confidence_head_inputs(cfg)
    hd = torch.from_numpy(h).cuda()
    wd = torch.from_numpy(w).cuda()
    dc = ds.dspark_draft_sample_confidence(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], hd, wd,
                                           seed, 0)
    d0 = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, 0)
    v = ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], dc["x"], dc["lse"], dc["qx"],
                         dev["temperature"], seed, 0)

    def step_conf(rid):
        ds.dspark_draft_sample_confidence(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], hd, wd,
                                          seed, rid, out=dc)
        ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], dc["x"], dc["lse"], dc["qx"],
                         dev["temperature"], seed, rid, out=v)

    def step_plain(rid):
        ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, rid, out=d0)
        ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d0["x"], d0["lse"], d0["qx"],
                         dev["temperature"], seed, rid, out=v)

    ms_plain = _events_ms(torch, step_plain, reps, 5000)
    ms_conf = _events_ms(torch, step_conf, reps, 6000)
    red_plain = _profiled(torch, ds, lambda i: step_plain(7000 + i), reps)["draft_reduce"]
    red_conf = _profiled(torch, ds, lambda i: step_conf(8000 + i), reps)["draft_reduce"]
    from roundkit import np_of
    c = np_of(dc["conf"])
    return {"d": h.shape[2], "round_ms": round(ms_conf, 5), "round_ms_without": round(ms_plain, 5),
            "draft_reduce_us": round(red_conf, 2), "draft_reduce_us_without": round(red_plain, 2),
            "mean_c": round(float(c.mean()), 4)}


def _rnn_head(torch, ds, S, cfg, dev, td, ed, seed, reps, d):
    """The round with the RNN head in place of the Markov head (hidden width
    d, synthetic h and Wgco): round time; the h-part product's time and MFMA
    rate (2 B gamma d 3r flops, once a round) and the per-position gate
    kernel's (2 B 2r 3r flops a launch; 2 B (2r + d) 3r when the h part is
    not precomputed)."""
    import numpy as np
    from roundkit import np_of
    h, _ = S.confidence_head_inputs(cfg, d)
    bits, _ = S.rnn_head_weights(cfg, d)
    hd = torch.from_numpy(h).cuda()
    wg = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    g = ds.dspark_draft_sample_rnn(dev["U"], dev["W1"], dev["W2"], wg, dev["anchor"], dev["temperature"], hd, seed, 0)
    v = ds.dspark_verify_rnn(td, ed, dev["U"], g["e"], dev["W2"], dev["anchor"], g["x"], g["lse"], g["qx"],
                             dev["temperature"], seed, 0)

    def step(rid):
        ds.dspark_draft_sample_rnn(dev["U"], dev["W1"], dev["W2"], wg, dev["anchor"], dev["temperature"], hd, seed,
                                   rid, out=g)
        ds.dspark_verify_rnn(td, ed, dev["U"], g["e"], dev["W2"], dev["anchor"], g["x"], g["lse"], g["qx"],
                             dev["temperature"], seed, rid, out=v)

    for i in range(20):
        step(9000 + i)
    ms = _events_ms(torch, step, reps, 9100)
    ph = _profiled(torch, ds, lambda i: step(9300 + i), reps)
    B, r, d = cfg.B, cfg.r, h.shape[2]
    pus = ph.get("rnn_hproj", 0.0)
    flops = 2.0 * B * (2 * r + (0 if pus > 0 else d)) * 3 * r
    pflops = 2.0 * B * cfg.gamma * d * 3 * r
    us = ph.get("rnn_gate", 0.0)
    return {"d": d, "round_ms": round(ms, 5), "rnn_hproj_us": round(pus, 2),
            "rnn_hproj_tflops": round(pflops / (pus * 1e-6) / 1e12, 1) if pus > 0 else None,
            "rnn_gate_us": round(us, 2),
            "rnn_gate_tflops": round(flops / (us * 1e-6) / 1e12, 1) if us > 0 else None,
            "draft_step_us": round(ph.get("draft_step", 0.0), 2), "draft_reduce_us": round(ph.get("draft_reduce", 0.0), 2),
            "emitted_per_round": int(np_of(v["n"]).sum()) + B}


def _sts_fit(torch, ds, S, reps=10):
    """Sequential temperature scaling of the head from 200,000 synthetic
    calibration samples (gamma 5, 76 grid temperatures 0.25..4, 15 bins):
    time per fit call."""
    import numpy as np
    c, n = S.sts_samples(200_000, [2.0, 0.5, 1.0, 1.5, 0.75], seed=1)
    grid = torch.from_numpy(np.round(np.arange(0.25, 4.0001, 0.05), 2).astype(np.float32)).cuda()
    cd, nd = torch.from_numpy(c).cuda(), torch.from_numpy(n).cuda()
    out = ds.dspark_sts_fit(cd, nd, grid)
    ws = torch.empty(ds.dspark_sts_workspace_size(len(c), c.shape[1], grid.numel(), 15), dtype=torch.uint8,
                     device="cuda")
    ms = _events_ms(torch, lambda i: ds.dspark_sts_fit(cd, nd, grid, workspace=ws), reps, 0)
    ph = _profiled(torch, ds, lambda i: ds.dspark_sts_fit(cd, nd, grid, workspace=ws), reps)
    return {"samples": len(c), "gamma": c.shape[1], "grid": grid.numel(), "bins": 15, "call_ms": round(ms, 4),
            "sts_hist_us": round(ph.get("sts_hist", 0.0), 2), "sts_pick_us": round(ph.get("sts_pick", 0.0), 2),
            "tau": [round(float(t), 2) for t in out["tau"].cpu()]}


def _acceptance(torch, ds, dev, td, ed, d, rnd, B, gamma, V, r, reps):
    """The acceptance-probability labelling pass over every verified position
    of the round: time per call and the HBM fractions of its two streaming
    kernels (algorithmic bytes: the row statistics read every verified target
    row; the accepted mass reads the sampled rows' target and U_k rows and W2
    once -- its workgroups of 256 rows each walk W2 again, from the caches)."""
    import numpy as np
    from roundkit import np_of
    alpha = ds.dspark_acceptance(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"],
                                 dev["temperature"])

    def call(i):
        ds.dspark_acceptance(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"],
                             dev["temperature"], out=alpha)

    for i in range(5):
        call(i)
    ms = _events_ms(torch, call, reps, 0)
    ph = _profiled(torch, ds, call, reps)
    ell = np_of(ed)
    sampled = np.asarray(rnd.temperature) > 0
    rows = int(ell.sum())
    srows = int(ell[sampled].sum())
    row = V * 4
    out = {"call_ms": round(ms, 4), "rows": rows, "sampled_rows": srows,
           "phases_us": {k: round(v, 2) for k, v in ph.items()}}
    for name, nbytes in (("accept_rowstats", rows * row), ("accept_mass", 2 * srows * row + V * r * 2)):
        us = ph.get(name, 0.0)
        if us > 0:
            gbs = nbytes / (us * 1e-6) / 1e9
            out[name] = {"bytes": nbytes, "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    a = np_of(alpha)
    out["mean_alpha_sampled"] = round(float(np.nanmean(a[sampled])), 4)
    return out


def _draft_bytes(B, V, r, wbytes):
    """Algorithmic bytes of one draft step: U_k, W2, the gathered W1 rows."""
    return B * V * 4 + V * r * wbytes + B * r * wbytes


def _measure_config(torch, ds, S, label, cfg, rnd, ell, reps, warm, copies):
    """One configuration: round 0 against the oracle on every request (the
    oracle timed on this host's cores), then `reps` rounds timed after `warm`
    warmup rounds, taking U and the target from `copies` copies in turn, then
    per-kernel event times over `reps` more rounds with their outcome counts.
    Returns the figures and the count of eligible requests that differ."""
    import numpy as np
    from roundkit import compare_draft, compare_verify, np_of, oracle_round, to_device
    dev = to_device(rnd)
    target = rnd.target_packed(ell)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    seed = cfg.seed
    d = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, 0,
                               margin=True)
    v = ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"], d["qx"],
                         dev["temperature"], seed, 0, diag=True, resid=True)
    torch.cuda.synchronize()
    gd = {k: np_of(t) for k, t in d.items() if k != "workspace"}
    gv = {k: np_of(t) for k, t in v.items() if k != "workspace"}
    t0 = time.time()
    od, ov = oracle_round(rnd, target, ell, seed, 0)
    cpu_s = time.time() - t0
    cd = compare_draft(gd, od, strict=False)
    cv = compare_verify(gv, od, ov, rnd.temperature, ell, strict=False)
    bad = int(cd.mismatch[cd.eligible].sum()) + int(cv.mismatch[cv.eligible].sum())
    Us = [dev["U"]] + [dev["U"].clone() for _ in range(copies - 1)]
    Ts = [td] + [td.clone() for _ in range(copies - 1)]
    dr = {k: d[k] for k in ("x", "lse", "qx", "workspace")}
    vr = {k: v[k] for k in ("n", "tokens", "offsets", "workspace")}

    def step(rid):
        U_r, t_r = Us[rid % copies], Ts[rid % copies]
        ds.dspark_draft_sample(U_r, dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, rid, out=dr)
        ds.dspark_verify(t_r, ed, U_r, dev["W1"], dev["W2"], dev["anchor"], dr["x"], dr["lse"], dr["qx"],
                         dev["temperature"], seed, rid, out=vr)

    for i in range(warm):
        step(100 + i)
    ms = _events_ms(torch, step, reps, 1000)
    add, mean = _outcome_counter(torch, dev["temperature"], ed)
    torch.cuda.synchronize()
    ds.dspark_profile_reset()
    ds.dspark_profile_enable(True)
    for i in range(reps):
        step(2000 + i)
        add(vr["n"])
    torch.cuda.synchronize()
    ds.dspark_profile_collect()
    ds.dspark_profile_enable(False)
    phases = {k: {"launches": n, "avg_us": 1e3 * t / max(1, n)} for k, (n, t) in ds.dspark_profile_read().items()
              if n > 0}
    wbytes = 2 if cfg.wdtype == "bf16" else 4
    res = {"B": cfg.B, "gamma": cfg.gamma, "V": cfg.V, "r": cfg.r, "weights": cfg.wdtype,
           "ell_mean": round(float(ell.mean()), 3), "round_ms": round(ms, 5),
           "drafted_positions_per_s": round(cfg.B * cfg.gamma / (ms * 1e-3), 1),
           "phases_us": {k: round(p["avg_us"], 2) for k, p in phases.items()}}
    if "draft_step" in phases:
        us = phases["draft_step"]["avg_us"]
        gbs = _draft_bytes(cfg.B, cfg.V, cfg.r, wbytes) / (us * 1e-6) / 1e9
        res["draft_step"] = {"bytes": _draft_bytes(cfg.B, cfg.V, cfg.r, wbytes), "gbs": round(gbs, 1),
                             "frac": round(gbs / HBM_PEAK_GBS, 4)}
    res["logit_passes"] = _logit_passes(phases, mean(), cfg.B, cfg.V, cfg.r)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    cores = int(os.environ.get("OMP_NUM_THREADS", cores))
    res["oracle"] = {"seconds": round(cpu_s, 3), "cores": cores,
                     "drafted_positions_per_s": round(cfg.B * cfg.gamma / cpu_s, 2),
                     "sample": "round 0 of the same inputs, every request: fp64 draft + verify"}
    res["parity"] = {"draft": cd.report(), "verify": cv.report(), "eligible_mismatches": bad}
    res["input_copies"] = copies
    del Us, Ts, dev, td, d, v, dr, vr
    torch.cuda.empty_cache()
    return res, bad


def _configs(torch, ds, S, reps):
    """Every configuration other than the headline one, each parity-gated."""
    import numpy as np
    out, bad = {}, 0
    for name in ("tiny", "dspark5", "long"):
        cfg = S.CONFIGS[name]
        rnd = S.make_round(cfg)
        ell = np.full(cfg.B, cfg.gamma, np.int32)
        r, b = _measure_config(torch, ds, S, name, cfg, rnd, ell, reps, 10, 1 if name == "tiny" else 3)
        out[name] = r
        bad += b
        print(f"# config {name}: {r['round_ms']} ms a round, parity {r['parity']['verify']}", file=sys.stderr,
              flush=True)
    # the scheduled batch: the scheduler's literal choice at rho = 0.2 (ell = 0
    # for every request at this cost curve), and the supplement that schedules
    # 256 groups of 4 requests independently
    cfg = S.CONFIGS["sched"]
    rnd = S.make_round(cfg)
    sps = S.sps_table_toy(0.2, cfg.B * (1 + cfg.gamma) + 1)
    t0 = time.perf_counter()
    ell, theta, tau, bsz = ds.dspark_schedule(rnd.c, sps)
    sched_us = (time.perf_counter() - t0) * 1e6
    ell = np.asarray(ell, np.int32)
    ell_g = np.concatenate([ds.dspark_schedule(rnd.c[4 * g:4 * g + 4], S.sps_table_toy(0.2, 25))[0]
                            for g in range(cfg.B // 4)]).astype(np.int32)
    for tag, e in (("sched_literal", ell), ("sched_groups4", ell_g)):
        r, b = _measure_config(torch, ds, S, tag, cfg, rnd, e, reps, 10, 3)
        r["scheduler"] = {"rho": 0.2, "ell_histogram": np.bincount(e, minlength=cfg.gamma + 1).tolist()}
        if tag == "sched_literal":
            r["scheduler"]["host_us_first_call"] = round(sched_us, 1)
        out[tag] = r
        bad += b
        print(f"# config {tag}: {r['round_ms']} ms a round, parity {r['parity']['verify']}", file=sys.stderr,
              flush=True)
    return out, bad


def _draft_step_cold(torch, ds, dev, B, gamma, V, r, seed, reps=20):
    """The draft step with its inputs evicted from the caches: a 512 MiB
    read before each launch.  Per-step: a one-position draft of U's first
    position (U_1, W2 and the gathered W1 rows all come from HBM).  Per round:
    the whole draft with the caches flushed before each round (W2 warm from
    the second position on, as between the positions of a served round)."""
    evict = _Evict(torch)
    U1 = dev["U"][:, :1, :].contiguous()
    d1 = ds.dspark_draft_sample(U1, dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, 0)
    dk = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, 0)
    out = {}
    for tag, U_, dd in (("step", U1, d1), ("round", dev["U"], dk)):
        torch.cuda.synchronize()
        ds.dspark_profile_reset()
        ds.dspark_profile_enable(True)
        for i in range(reps):
            evict()
            ds.dspark_draft_sample(U_, dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, i, out=dd)
        torch.cuda.synchronize()
        ds.dspark_profile_collect()
        ds.dspark_profile_enable(False)
        n, ms = ds.dspark_profile_read()["draft_step"]
        us = 1e3 * ms / n
        gbs = _draft_bytes(B, V, r, 2) / (us * 1e-6) / 1e9
        out[tag] = {"avg_us": round(us, 2), "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del evict, U1
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a round takes about 0.4 ms: a hundred warmup rounds bring the clocks to
    # their sustained level (five leave the timed rounds about 5% slower)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg (and the parity gate)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configurations")
    ap.add_argument("--rounds", type=int, default=60, help="rounds timed one by one for the round-time distribution")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary measurements (bias product, cold step, heads, scheduler, calibration)")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only time the bias product alone (warm and cold) and print its JSON (for counter runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-mebibyte device buffer 5 times (calibrates HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.empty(n // 4, dtype=torch.float32, device="cuda").uniform_()  # not an elementwise kernel
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)  # an elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the round is data-parallel over requests; sharding is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_sampling_verification_02_amd as ds
    import synth_inputs as S
    from roundkit import compare_draft, compare_verify, np_of, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    ds.load_library()
    cfg = S.CONFIGS["large"]
    B, gamma, V, r = cfg.B, cfg.gamma, cfg.V, cfg.r
    t0 = time.time()
    rnd = S.make_round(cfg)
    ell = np.full(B, gamma, np.int32)
    target = rnd.target_packed(ell)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = to_device(rnd)
    td = torch.from_numpy(target).cuda()
    ed = torch.from_numpy(ell).cuda()
    seed = cfg.seed
    if args.gemm_only:
        print(json.dumps({"bias_gemm_alone": _bias_gemm_alone(torch, ds, dev, B, V, r)}), flush=True)
        return

    # round 0, compared with the oracle below
    d = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, 0,
                               margin=True)
    v = ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"], d["qx"],
                         dev["temperature"], seed, 0, diag=True, resid=True)
    torch.cuda.synchronize()
    gd0 = {k: np_of(t) for k, t in d.items() if k != "workspace"}
    gv0 = {k: np_of(t) for k, t in v.items() if k != "workspace"}

    result_cpu, parity, bad = None, None, 0
    if not args.no_cpu:
        from roundkit import oracle_round
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count()
        cores = int(os.environ.get("OMP_NUM_THREADS", cores))
        t0 = time.time()
        od, ov = oracle_round(rnd, target, ell, seed, 0)
        cpu_s = time.time() - t0
        cd = compare_draft(gd0, od, strict=False)
        cv = compare_verify(gv0, od, ov, rnd.temperature, ell, strict=False)
        bad += int(cv.mismatch[cv.eligible].sum()) + int(cd.mismatch[cd.eligible].sum())
        result_cpu = {"value": round(B * gamma / cpu_s, 2), "unit": "drafted positions/s", "cores": cores,
                      "kind": "oracle",
                      "sample": f"one full round of the same workload (B={B}, gamma={gamma}, V={V}): "
                                f"fp64 draft + verify, {cpu_s:.1f}s"}
        result_cpu["one_thread"] = _oracle_one_thread(rnd, target, ell, seed, gamma, oracle_round)
        parity = {"draft": cd.report(), "verify": cv.report(),
                  "eligible_mismatches": int(cv.mismatch[cv.eligible].sum()) + int(cd.mismatch[cd.eligible].sum())}
        print(f"# oracle: {cpu_s:.1f}s, parity {cv.report()}", file=sys.stderr, flush=True)

    # every other configuration, parity-gated on every request
    configs = None
    if not args.no_cpu and not args.no_configs:
        configs, cbad = _configs(torch, ds, S, 30)
        bad += cbad

    # Each timed round takes its U and target from one of three identical
    # copies in turn, so that no round finds the logit rows of the round
    # before in the caches (about 1.5 GB of rows a copy); the weights are
    # shared, as in serving, where W1 and W2 stay resident from round to round.
    Us = [dev["U"]] + [dev["U"].clone() for _ in range(INPUT_COPIES - 1)]
    Ts = [td] + [td.clone() for _ in range(INPUT_COPIES - 1)]
    d = {"x": d["x"], "lse": d["lse"], "qx": d["qx"], "workspace": d["workspace"]}
    v = {k: v[k] for k in ("n", "tokens", "offsets", "workspace")}

    def step(rid):
        U_r, t_r = Us[rid % INPUT_COPIES], Ts[rid % INPUT_COPIES]
        ds.dspark_draft_sample(U_r, dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, rid, out=d)
        ds.dspark_verify(t_r, ed, U_r, dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"], d["qx"],
                         dev["temperature"], seed, rid, out=v)

    # secondary GPU measurements (before the timed region)
    gemm = cold = sched = conf = accept = rnn = rnn_wide = sts = None
    if not args.no_secondary:
        gemm = _bias_gemm_alone(torch, ds, dev, B, V, r)
        cold = _draft_step_cold(torch, ds, dev, B, gamma, V, r, seed)
        sched = _schedule_time(ds, S)
        conf = _confidence_head(torch, ds, S, cfg, dev, td, ed, seed, 30)
        accept = _acceptance(torch, ds, dev, td, ed, d, rnd, B, gamma, V, r, 20)
        rnn = _rnn_head(torch, ds, S, cfg, dev, td, ed, seed, 30, S.DEFAULT_HIDDEN)
        rnn_wide = _rnn_head(torch, ds, S, cfg, dev, td, ed, seed, 30, 4 * S.DEFAULT_HIDDEN)
        sts = _sts_fit(torch, ds, S)

    # single-round times (also the rounds that lead into the timed region,
    # after the heavier secondary work)
    round_dist = _round_distribution(torch, step, args.rounds, 3000)

    # the timed region: W warmup rounds, then K rounds between two events
    for i in range(args.warmup):
        step(1 + i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(1000 + i)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    emitted = int(np_of(v["n"]).sum()) + B

    # instrumented pass: per-kernel HIP events on the launch stream, and the
    # rounds' outcomes (rows the walk read, draws of each kind)
    add, mean = _outcome_counter(torch, dev["temperature"], ed)
    ds.dspark_profile_reset()
    ds.dspark_profile_enable(True)
    for i in range(args.steps):
        step(2000 + i)
        add(v["n"])
    torch.cuda.synchronize()
    ds.dspark_profile_collect()
    ds.dspark_profile_enable(False)
    prof = ds.dspark_profile_read()
    phases = {k: {"launches": n, "avg_us": 1e3 * ms / max(1, n)} for k, (n, ms) in prof.items() if n > 0}
    outcome = mean()

    drafted = B * gamma
    value = drafted / (ms_step * 1e-3)
    # dominant kernel: draft_step (gamma launches per step)
    ds_avg_s = phases["draft_step"]["avg_us"] * 1e-6
    bytes_per_launch = _draft_bytes(B, V, r, 2)  # U_k slice, W2, gathered W1 rows
    achieved = bytes_per_launch / ds_avg_s / 1e9
    flops_per_launch = 2.0 * B * r * V
    traffic = _traffic_from_counters(bytes_per_launch)
    roofline = {"kernel": "draft_step", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": bytes_per_launch,
                "frac_inputs_evicted": cold["step"]["frac"] if cold else None,
                "mfma_bf16_tflops": round(flops_per_launch / ds_avg_s / 1e12, 1),
                "mfma_frac": round(flops_per_launch / ds_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "kernel_source_hash": _kernel_hash()}

    logit = _logit_passes(phases, outcome, B, V, r)

    result = {
        "metric": "draft+verify positions/sec at B=256 gamma=5 V=129k; % of HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "drafted positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded normal logits and bf16 Markov factors; no trained weights)",
        "config": {"workload": "large-batch round: B=256 gamma=5 V=129280 r=256 bf16 W1/W2, f32 U/target, "
                               "10% greedy, ell=gamma", "B": B, "gamma": gamma, "V": V, "r": r,
                   "input_copies": INPUT_COPIES, "parallelism": "single-gpu"},
        "secondary": {"verified_positions_per_s": round(B * (gamma + 1) / (ms_step * 1e-3), 1),
                      "emitted_tokens_per_s": round(emitted / (ms_step * 1e-3), 1),
                      "phases_us": {k: round(p["avg_us"], 2) for k, p in phases.items()},
                      "round_ms": round_dist,
                      "draft_step_inputs_evicted": cold,
                      "bias_gemm_alone": gemm,
                      "logit_passes": logit,
                      "configs": configs,
                      "schedule": sched,
                      "confidence_head": conf,
                      "acceptance": accept,
                      "rnn_head": rnn, "rnn_head_wide": rnn_wide,
                      "sts_fit": sts},
        "roofline": roofline,
    }
    if result_cpu is not None:
        result["cpu_baseline"] = result_cpu
        result["parity"] = parity
    print(json.dumps(result), flush=True)
    if bad:
        print("parity gate failed: eligible requests differ from the oracle", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
