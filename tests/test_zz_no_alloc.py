"""The allocation-free draft entry point against dspark_draft_sample.

dspark_draft_sample_noalloc takes its scratch from the library's fixed
per-device array instead of a caller workspace.  Its outputs must be the bits
dspark_draft_sample writes for the same inputs.  Two calls in a row, the
second with a smaller input, so that the second call finds the first one's
contents in the shared array: the draft's scratch is fully rewritten before
it is read, so they must not matter."""
import numpy as np
import pytest

import synth_inputs as S
from roundkit import np_of, to_device

pytestmark = pytest.mark.gpu


def _run_pair(ds, dev, seed, round_id):
    # both entry points on the same inputs; outputs preallocated by the first
    ref = ds.dspark_draft_sample(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed, round_id,
                                 margin=True)
    out = {k: v.clone().fill_(-7) for k, v in ref.items() if k != "workspace"}
    got = ds.dspark_draft_sample_noalloc(dev["U"], dev["W1"], dev["W2"], dev["anchor"], dev["temperature"], seed,
                                         round_id, margin=True, out=out)
    return {k: np_of(v) for k, v in ref.items() if k != "workspace"}, {k: np_of(v) for k, v in got.items()}


def test_noalloc_draft_matches_workspace_draft_on_two_calls():
    import torch
    import draft_sampling_verification_02_amd as ds
    assert torch.cuda.is_available()
    ds.load_library()
    calls = [("large", {}), ("tiny", dict(B=3))]  # the second input is smaller in every dimension
    for name, over in calls:
        cfg = S.CONFIGS[name].with_(**over)
        print(f"noalloc draft: {name} B={cfg.B} gamma={cfg.gamma} V={cfg.V} r={cfg.r}", flush=True)
        rnd = S.make_round(cfg)
        dev = to_device(rnd)
        ref, got = _run_pair(ds, dev, cfg.seed, 5)
        torch.cuda.synchronize()
        for k in ("x", "lse", "qx", "margin"):
            assert ref[k].shape == got[k].shape, k
            assert np.array_equal(ref[k].view(np.uint32), got[k].view(np.uint32)), (name, k)
        assert (ref["x"] >= 0).all() and (ref["x"] < cfg.V).all()


def test_noalloc_draft_rejects_sizes_beyond_its_scratch():
    import torch
    import draft_sampling_verification_02_amd as ds
    lib = ds.load_library()
    B, gamma, V, r = 13697, 1, 129280, 256
    assert lib.dspark_draft_workspace_size(B, gamma, V, r) > ds.DSPARK_NOALLOC_SCRATCH_BYTES
    # tiny real buffers: the call must refuse before it reads any of them
    f = torch.zeros(16, device="cuda")
    i = torch.zeros(16, dtype=torch.int32, device="cuda")
    w = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    st = lib.dspark_draft_sample_noalloc(ds._ptr(f), ds._ptr(w), ds._ptr(w), 0, ds._ptr(i), ds._ptr(f), B, gamma, V, r,
                                         1, 0, ds._ptr(i), ds._ptr(f), ds._ptr(f), None, ds._stream_ptr(None))
    assert st == ds.DSPARK_ERR_SCRATCH
