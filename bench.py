#!/usr/bin/env python3
"""Benchmark: one DSpark draft-and-verify round per step on one MI355X.

Workload: the large-batch round -- B = 256 requests, gamma = 5 block
positions, V = 129,280 vocabulary, rank r = 256 bf16 Markov factors, float32
base and target logits, 10% greedy requests, every drafted position verified
(ell = gamma).  Inputs are seeded synthetic data already resident in HBM when
the timed region starts.  A step is dspark_draft_sample + dspark_verify over
the whole batch; round_id advances every step.

The printed JSON line carries the headline throughput (drafted positions per
second), the dominant kernel's roofline figures measured with HIP events on
the launch stream, and the CPU oracle timed on this host on one full round of
the same workload (which also gates parity: eligible requests must match).

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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg (and the parity gate)")
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

    d = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, 0,
                               margin=True)
    v = ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"], d["qx"],
                         dev["temperature"], seed, 0, diag=True, resid=True)
    torch.cuda.synchronize()
    gd0 = {k: np_of(t) for k, t in d.items() if k != "workspace"}
    gv0 = {k: np_of(t) for k, t in v.items() if k != "workspace"}

    def step(rid):
        ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, rid,
                               out=d)
        ds.dspark_verify(td, ed, dev["U"], dev["W1"], dev["W2"], dev["anchor"], d["x"], d["lse"], d["qx"],
                         dev["temperature"], seed, rid, out=v)

    # plain timed region
    out_plain = {"x": d["x"], "lse": d["lse"], "qx": d["qx"], "workspace": d["workspace"]}
    d = out_plain
    v = {k: v[k] for k in ("n", "tokens", "offsets", "workspace")}
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

    # instrumented pass: per-kernel HIP events on the launch stream
    ds.dspark_profile_reset()
    ds.dspark_profile_enable(True)
    for i in range(args.steps):
        step(2000 + i)
    torch.cuda.synchronize()
    ds.dspark_profile_collect()
    ds.dspark_profile_enable(False)
    prof = ds.dspark_profile_read()
    phases = {k: {"launches": n, "avg_us": 1e3 * ms / max(1, n)} for k, (n, ms) in prof.items()}

    drafted = B * gamma
    value = drafted / (ms_step * 1e-3)
    # dominant kernel: draft_step (gamma launches per step)
    ds_avg_s = phases["draft_step"]["avg_us"] * 1e-6
    bytes_per_launch = B * V * 4 + V * r * 2 + B * r * 2  # U_k slice, W2, gathered W1 rows
    achieved = bytes_per_launch / ds_avg_s / 1e9
    flops_per_launch = 2.0 * B * r * V
    traffic = _traffic_from_counters(bytes_per_launch)
    roofline = {"kernel": "draft_step", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": bytes_per_launch,
                "mfma_bf16_tflops": round(flops_per_launch / ds_avg_s / 1e12, 1),
                "mfma_frac": round(flops_per_launch / ds_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "kernel_source_hash": _kernel_hash()}

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
                   "parallelism": "single-gpu"},
        "secondary": {"verified_positions_per_s": round(B * (gamma + 1) / (ms_step * 1e-3), 1),
                      "emitted_tokens_per_s": round(emitted / (ms_step * 1e-3), 1),
                      "phases_us": {k: round(p["avg_us"], 2) for k, p in phases.items()}},
        "roofline": roofline,
    }

    if not args.no_cpu:
        import oracle
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
        result["cpu_baseline"] = {"value": round(drafted / cpu_s, 2), "unit": "drafted positions/s",
                                  "cores": cores, "kind": "oracle",
                                  "sample": f"one full round of the same workload (B={B}, gamma={gamma}, "
                                            f"V={V}): fp64 draft + verify, {cpu_s:.1f}s"}
        result["parity"] = {"draft": cd.report(), "verify": cv.report(),
                            "eligible_mismatches": int(cv.mismatch[cv.eligible].sum()) + int(cd.mismatch[cd.eligible].sum())}
        if cv.mismatch[cv.eligible].any() or cd.mismatch[cd.eligible].any():
            print(json.dumps(result), flush=True)
            print("parity gate failed: eligible requests differ from the oracle", file=sys.stderr)
            sys.exit(1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
