"""Python binding of libdspark.so, the MI355X (gfx950) library for one DSpark
draft-and-verify round.

Argument marshalling only: every step of the round runs in the library's HIP
kernels (or, for the scheduler, its host C++).  Device arrays are torch
tensors on the current HIP device, passed by pointer together with torch's
current stream; host arrays (scheduler) are numpy arrays.  The functions
carry the C entry points' names.  A missing or unloadable library raises
immediately: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "DSparkError", "load_library", "DSPARK_BF16", "DSPARK_F32",
    "dspark_version", "dspark_status_string",
    "dspark_draft_workspace_size", "dspark_draft_sample",
    "dspark_verify_workspace_size", "dspark_verify", "dspark_verify_check",
    "dspark_schedule", "dspark_debug_random_words", "dspark_debug_gumbel", "dspark_debug_bias_gemm",
    "dspark_profile_enable", "dspark_profile_collect", "dspark_profile_read", "dspark_profile_reset",
]

DSPARK_OK = 0
DSPARK_ERR_ARG = -1
DSPARK_ERR_UNSUPPORTED = -2
DSPARK_ERR_WORKSPACE = -3
DSPARK_ERR_HIP = -4
DSPARK_ERR_DEVICE_INPUT = -5
DSPARK_ERR_SCRATCH = -6
DSPARK_NOALLOC_SCRATCH_BYTES = 8 << 20  # the allocation-free draft's fixed scratch (include/dspark.h)
DSPARK_BF16 = 0
DSPARK_F32 = 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdspark.so")

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_u64 = ctypes.c_uint64
_c_size = ctypes.c_size_t
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)

_lib = None


class DSparkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dspark_status_string(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdspark.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libdspark.so not built at {path}; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    sig = {
        "dspark_version": ([], _c_int),
        "dspark_status_string": ([_c_int], ctypes.c_char_p),
        "dspark_draft_workspace_size": ([_c_int] * 4, _c_size),
        "dspark_draft_sample": ([_c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                 _c_int, _c_int, _c_int, _c_int, _c_u64, _c_u64,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_draft_sample_noalloc": ([_c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                         _c_int, _c_int, _c_int, _c_int, _c_u64, _c_u64,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p], _c_int),
        "dspark_draft_sample_confidence": ([_c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                            _c_int, _c_int, _c_int, _c_int, _c_u64, _c_u64,
                                            _c_void_p, _c_void_p, _c_int, _c_void_p,
                                            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                            _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_draft_rnn_workspace_size": ([_c_int] * 5, _c_size),
        "dspark_draft_sample_rnn": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                     _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_u64, _c_u64,
                                     _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                     _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_sts_workspace_size": ([_c_int] * 4, _c_size),
        "dspark_sts_fit": ([_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_void_p, _c_int, _c_int,
                            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_verify_workspace_size": ([_c_int] * 4, _c_size),
        "dspark_verify": ([_c_void_p, _c_int, _c_void_p, _c_void_p,
                           _c_void_p, _c_void_p, _c_void_p, _c_int,
                           _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _c_int, _c_int, _c_int, _c_int, _c_u64, _c_u64,
                           _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_verify_check": ([_c_void_p, _c_void_p], _c_int),
        "dspark_verify_rnn": ([_c_void_p, _c_int, _c_void_p, _c_void_p,
                               _c_void_p, _c_void_p, _c_void_p, _c_int,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _c_int, _c_int, _c_int, _c_int, _c_u64, _c_u64,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_acceptance_rnn": ([_c_void_p, _c_int, _c_void_p, _c_void_p,
                                   _c_void_p, _c_void_p, _c_void_p, _c_int,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_int, _c_int, _c_int, _c_int,
                                   _c_void_p, _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_acceptance_workspace_size": ([_c_int] * 4, _c_size),
        "dspark_acceptance": ([_c_void_p, _c_int, _c_void_p, _c_void_p,
                               _c_void_p, _c_void_p, _c_void_p, _c_int,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _c_int, _c_int, _c_int, _c_int,
                               _c_void_p, _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_schedule": ([_f64p, _c_int, _c_int, _f64p, _c_int, _i32p, _f64p, _f64p, _i32p], _c_int),
        "dspark_history_capacity": ([_i32p, _i32p, _c_int, _c_int, _c_int, ctypes.POINTER(ctypes.c_int64)], _c_int),
        "dspark_schedule_capacity": ([_f64p, _c_int, _c_int, ctypes.c_int64, _i32p, _f64p, _i32p], _c_int),
        "dspark_debug_random_words": ([_c_u64, _c_u64, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_void_p, _c_void_p], _c_int),
        "dspark_debug_gumbel": ([_c_void_p, _c_int, _c_void_p, _c_void_p], _c_int),
        "dspark_debug_bias_gemm": ([_c_void_p, _c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_void_p,
                                    _c_void_p, _c_size, _c_void_p], _c_int),
        "dspark_profile_enable": ([_c_int], _c_int),
        "dspark_profile_collect": ([], _c_int),
        "dspark_profile_count": ([], _c_int),
        "dspark_profile_get": ([_c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int64),
                                _f64p], _c_int),
        "dspark_profile_reset": ([], _c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != DSPARK_OK:
        raise DSparkError(status, where)


def dspark_version() -> int:
    return load_library().dspark_version()


def dspark_status_string(status: int) -> str:
    return load_library().dspark_status_string(int(status)).decode()


# ---------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _weights(W1, W2, device):
    torch = _torch()
    if W1.dtype == torch.bfloat16 and W2.dtype == torch.bfloat16:
        wdt = DSPARK_BF16
    elif W1.dtype == torch.float32 and W2.dtype == torch.float32:
        wdt = DSPARK_F32
    else:
        raise TypeError("W1/W2: both bfloat16 or both float32")
    if W1.shape != W2.shape or W1.dim() != 2:
        raise ValueError("W1/W2: equal [V, r] shapes")
    for n, t in (("W1", W1), ("W2", W2)):
        _need(t, n, t.dtype, None, device)
    return wdt


def dspark_draft_workspace_size(B: int, gamma: int, V: int, r: int) -> int:
    return load_library().dspark_draft_workspace_size(B, gamma, V, r)


def dspark_verify_workspace_size(B: int, gamma: int, V: int, r: int) -> int:
    return load_library().dspark_verify_workspace_size(B, gamma, V, r)


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
    return workspace


def _draft_outputs(B, gamma, dev, margin, conf, out):
    torch = _torch()
    if out is None:
        out = {"x": torch.empty((B, gamma), dtype=torch.int32, device=dev),
               "lse": torch.empty((B, gamma), dtype=torch.float32, device=dev),
               "qx": torch.empty((B, gamma), dtype=torch.float32, device=dev)}
        if margin:
            out["margin"] = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        if conf:
            out["conf"] = torch.empty((B, gamma), dtype=torch.float32, device=dev)
            out["survival"] = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    return out


def _draft_inputs(U, W1, W2, anchor, temperature):
    torch = _torch()
    dev = U.device
    B, gamma, V = U.shape
    _need(U, "U", torch.float32, (B, gamma, V), dev)
    wdt = _weights(W1, W2, dev)
    if W1.shape[0] != V:
        raise ValueError("W1/W2: first dimension must be V")
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    return dev, B, gamma, V, W1.shape[1], wdt


def dspark_draft_sample(U, W1, W2, anchor, temperature, seed: int, round_id: int, *,
                        margin: bool = False, out: dict | None = None, workspace=None, stream=None) -> dict:
    """Draft half of a round.  U [B, gamma, V] float32, W1/W2 [V, r] bf16 or
    float32, anchor [B] int32, temperature [B] float32 -- all on one HIP device.
    Returns {"x", "lse", "qx"[, "margin"], "workspace"}; pass ``out`` (a
    previous result) to reuse its buffers."""
    lib = load_library()
    dev, B, gamma, V, r, wdt = _draft_inputs(U, W1, W2, anchor, temperature)
    out = _draft_outputs(B, gamma, dev, margin, False, out)
    nbytes = lib.dspark_draft_workspace_size(B, gamma, V, r)
    if nbytes == 0:
        raise DSparkError(DSPARK_ERR_ARG, "dspark_draft_workspace_size")
    ws = _workspace(nbytes, dev, workspace if workspace is not None else out.get("workspace"))
    out["workspace"] = ws
    st = lib.dspark_draft_sample(_ptr(U), _ptr(W1), _ptr(W2), wdt, _ptr(anchor), _ptr(temperature),
                                 B, gamma, V, r, int(seed), int(round_id),
                                 _ptr(out["x"]), _ptr(out["lse"]), _ptr(out["qx"]), _ptr(out.get("margin")),
                                 _ptr(ws), ws.numel(), _stream_ptr(stream))
    _check(st, "dspark_draft_sample")
    return out


def dspark_draft_sample_noalloc(U, W1, W2, anchor, temperature, seed: int, round_id: int, *,
                                margin: bool = False, out: dict | None = None, stream=None) -> dict:
    """dspark_draft_sample without a workspace: the library's fixed per-device
    scratch serves instead, and the C call allocates nothing.  Pass ``out`` (a
    previous result) so that this wrapper allocates no outputs either.
    Returns {"x", "lse", "qx"[, "margin"]}."""
    lib = load_library()
    dev, B, gamma, V, r, wdt = _draft_inputs(U, W1, W2, anchor, temperature)
    out = _draft_outputs(B, gamma, dev, margin, False, out)
    st = lib.dspark_draft_sample_noalloc(_ptr(U), _ptr(W1), _ptr(W2), wdt, _ptr(anchor), _ptr(temperature),
                                         B, gamma, V, r, int(seed), int(round_id),
                                         _ptr(out["x"]), _ptr(out["lse"]), _ptr(out["qx"]), _ptr(out.get("margin")),
                                         _stream_ptr(stream))
    _check(st, "dspark_draft_sample_noalloc")
    return out


def dspark_draft_sample_confidence(U, W1, W2, anchor, temperature, hidden, conf_w, seed: int, round_id: int, *,
                                   conf_tau=None, margin: bool = False, out: dict | None = None, workspace=None,
                                   stream=None) -> dict:
    """dspark_draft_sample plus the confidence head c_k = sigmoid(conf_w .
    [h_k, W1[x_{k-1}]] / tau_k) and the survival products a_k = c_1...c_k.
    hidden [B, gamma, d] float32 (d may be 0), conf_w [d + r] float32,
    conf_tau [gamma] float32 or None (tau = 1; dspark_sts_fit's output).
    Returns the draft outputs plus {"conf", "survival"}."""
    torch = _torch()
    lib = load_library()
    dev, B, gamma, V, r, wdt = _draft_inputs(U, W1, W2, anchor, temperature)
    if hidden.dim() != 3 or tuple(hidden.shape[:2]) != (B, gamma):
        raise ValueError("hidden: [B, gamma, d]")
    d = hidden.shape[2]
    _need(hidden, "hidden", torch.float32, (B, gamma, d), dev)
    _need(conf_w, "conf_w", torch.float32, (d + r,), dev)
    if conf_tau is not None:
        _need(conf_tau, "conf_tau", torch.float32, (gamma,), dev)
    out = _draft_outputs(B, gamma, dev, margin, True, out)
    nbytes = lib.dspark_draft_workspace_size(B, gamma, V, r)
    if nbytes == 0:
        raise DSparkError(DSPARK_ERR_ARG, "dspark_draft_workspace_size")
    ws = _workspace(nbytes, dev, workspace if workspace is not None else out.get("workspace"))
    out["workspace"] = ws
    st = lib.dspark_draft_sample_confidence(
        _ptr(U), _ptr(W1), _ptr(W2), wdt, _ptr(anchor), _ptr(temperature), B, gamma, V, r, int(seed),
        int(round_id), _ptr(hidden) if d > 0 else None, _ptr(conf_w), d, _ptr(conf_tau),
        _ptr(out["x"]), _ptr(out["lse"]), _ptr(out["qx"]), _ptr(out.get("margin")),
        _ptr(out["conf"]), _ptr(out["survival"]), _ptr(ws), ws.numel(), _stream_ptr(stream))
    _check(st, "dspark_draft_sample_confidence")
    return out


def dspark_draft_rnn_workspace_size(B: int, gamma: int, V: int, r: int, d: int) -> int:
    return load_library().dspark_draft_rnn_workspace_size(B, gamma, V, r, d)


def dspark_draft_sample_rnn(U, W1, W2, Wgco, anchor, temperature, hidden, seed: int, round_id: int, *,
                            margin: bool = False, state: bool = False, out: dict | None = None, workspace=None,
                            stream=None) -> dict:
    """Draft half with the RNN head.  W1/W2 [V, r] and Wgco [3r, 2r + d]
    bfloat16, hidden [B, gamma, d] float32 (d a multiple of 32, may be 0).
    Returns the draft outputs plus {"e"} (the head's rows [B, gamma, r]
    bfloat16, for dspark_verify_rnn) [and {"state"} = s_gamma [B, r]]."""
    torch = _torch()
    lib = load_library()
    dev, B, gamma, V, r, wdt = _draft_inputs(U, W1, W2, anchor, temperature)
    if hidden.dim() != 3 or tuple(hidden.shape[:2]) != (B, gamma):
        raise ValueError("hidden: [B, gamma, d]")
    d = hidden.shape[2]
    _need(hidden, "hidden", torch.float32, (B, gamma, d), dev)
    _need(Wgco, "Wgco", W1.dtype, (3 * r, 2 * r + d), dev)
    out = _draft_outputs(B, gamma, dev, margin, False, out)
    if "e" not in out:
        out["e"] = torch.empty((B, gamma, r), dtype=torch.bfloat16, device=dev)
    if state and "state" not in out:
        out["state"] = torch.empty((B, r), dtype=torch.float32, device=dev)
    nbytes = lib.dspark_draft_rnn_workspace_size(B, gamma, V, r, d)
    if nbytes == 0:
        raise DSparkError(DSPARK_ERR_ARG, "dspark_draft_rnn_workspace_size")
    ws = _workspace(nbytes, dev, workspace if workspace is not None else out.get("workspace"))
    out["workspace"] = ws
    st = lib.dspark_draft_sample_rnn(
        _ptr(U), _ptr(W1), _ptr(W2), _ptr(Wgco), wdt, _ptr(anchor), _ptr(temperature),
        _ptr(hidden) if d > 0 else None, d, B, gamma, V, r, int(seed), int(round_id),
        _ptr(out["x"]), _ptr(out["lse"]), _ptr(out["qx"]), _ptr(out.get("margin")), _ptr(out["e"]),
        _ptr(out.get("state")), _ptr(ws), ws.numel(), _stream_ptr(stream))
    _check(st, "dspark_draft_sample_rnn")
    return out


def dspark_verify(target, ell, U, W1, W2, anchor, x, lse_q, qx, temperature, seed: int, round_id: int, *,
                  row_offsets=None, diag: bool = False, resid: bool = False, out_offsets: bool = True,
                  out: dict | None = None, workspace=None, stream=None) -> dict:
    """Verify half of a round.  target [rows, V] float32 packed per request
    (rows off_b .. off_b + ell_b), ell [B] int32, and the draft's inputs and
    outputs.  Returns {"n", "tokens"[, "offsets", "diag", "resid"], "workspace"}."""
    return _verify(target, ell, U, W1, W2, anchor, x, lse_q, qx, temperature, seed, round_id, None,
                   row_offsets, diag, resid, out_offsets, out, workspace, stream)


def dspark_verify_rnn(target, ell, U, head_rows, W2, anchor, x, lse_q, qx, temperature, seed: int, round_id: int, *,
                      row_offsets=None, diag: bool = False, resid: bool = False, out_offsets: bool = True,
                      out: dict | None = None, workspace=None, stream=None) -> dict:
    """dspark_verify for RNN-head drafts: q_k from head_rows [B, gamma, r]
    (the "e" output of dspark_draft_sample_rnn) instead of W1[x_{k-1}]."""
    torch = _torch()
    B, gamma, _ = U.shape
    _need(head_rows, "head_rows", W2.dtype, (B, gamma, W2.shape[1]), U.device)
    return _verify(target, ell, U, W2, W2, anchor, x, lse_q, qx, temperature, seed, round_id, head_rows,
                   row_offsets, diag, resid, out_offsets, out, workspace, stream)


def _verify(target, ell, U, W1, W2, anchor, x, lse_q, qx, temperature, seed, round_id, rows,
            row_offsets, diag, resid, out_offsets, out, workspace, stream):
    torch = _torch()
    lib = load_library()
    dev = U.device
    B, gamma, V = U.shape
    r = W1.shape[1]
    _need(U, "U", torch.float32, (B, gamma, V), dev)
    wdt = _weights(W1, W2, dev)
    if target.dim() != 2 or target.shape[1] != V:
        raise ValueError("target: [rows, V]")
    _need(target, "target", torch.float32, None, dev)
    _need(ell, "ell", torch.int32, (B,), dev)
    if row_offsets is not None:
        _need(row_offsets, "row_offsets", torch.int32, (B + 1,), dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(x, "x", torch.int32, (B, gamma), dev)
    _need(lse_q, "lse_q", torch.float32, (B, gamma), dev)
    _need(qx, "qx", torch.float32, (B, gamma), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    if out is None:
        out = {"n": torch.empty(B, dtype=torch.int32, device=dev),
               "tokens": torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)}
        if out_offsets:
            out["offsets"] = torch.empty(B + 1, dtype=torch.int32, device=dev)
        if diag:
            out["diag"] = torch.empty((B, gamma + 1, 2), dtype=torch.float32, device=dev)
        if resid:
            out["resid"] = torch.empty(B, dtype=torch.float32, device=dev)
    nbytes = lib.dspark_verify_workspace_size(B, gamma, V, r)
    if nbytes == 0:
        raise DSparkError(DSPARK_ERR_ARG, "dspark_verify_workspace_size")
    ws = _workspace(nbytes, dev, workspace if workspace is not None else out.get("workspace"))
    out["workspace"] = ws
    fn = lib.dspark_verify if rows is None else lib.dspark_verify_rnn
    st = fn(_ptr(target), target.shape[0], _ptr(ell), _ptr(row_offsets),
            _ptr(U), _ptr(W1 if rows is None else rows), _ptr(W2), wdt, _ptr(anchor), _ptr(x), _ptr(lse_q),
            _ptr(qx), _ptr(temperature), B, gamma, V, r, int(seed), int(round_id),
            _ptr(out["n"]), _ptr(out["tokens"]), _ptr(out.get("offsets")),
            _ptr(out.get("diag")), _ptr(out.get("resid")),
            _ptr(ws), ws.numel(), _stream_ptr(stream))
    _check(st, "dspark_verify" if rows is None else "dspark_verify_rnn")
    return out


def dspark_acceptance_workspace_size(B: int, gamma: int, V: int, r: int) -> int:
    return load_library().dspark_acceptance_workspace_size(B, gamma, V, r)


def dspark_acceptance(target, ell, U, W1, W2, anchor, x, lse_q, temperature, *, row_offsets=None,
                      out=None, workspace=None, stream=None):
    """Per-position acceptance probability alpha_k = sum_v min(p_k, q_k) of
    every verified position (NaN past ell).  Arguments as for dspark_verify.
    Returns alpha [B, gamma] float32 (``out`` if given)."""
    return _acceptance(target, ell, U, W1, W2, anchor, x, lse_q, temperature, None, row_offsets, out, workspace,
                       stream)


def dspark_acceptance_rnn(target, ell, U, head_rows, W2, anchor, x, lse_q, temperature, *, row_offsets=None,
                          out=None, workspace=None, stream=None):
    """dspark_acceptance for RNN-head drafts (q_k from head_rows)."""
    B, gamma, _ = U.shape
    _need(head_rows, "head_rows", W2.dtype, (B, gamma, W2.shape[1]), U.device)
    return _acceptance(target, ell, U, W2, W2, anchor, x, lse_q, temperature, head_rows, row_offsets, out,
                       workspace, stream)


def _acceptance(target, ell, U, W1, W2, anchor, x, lse_q, temperature, rows, row_offsets, out, workspace, stream):
    torch = _torch()
    lib = load_library()
    dev = U.device
    B, gamma, V = U.shape
    r = W1.shape[1]
    _need(U, "U", torch.float32, (B, gamma, V), dev)
    wdt = _weights(W1, W2, dev)
    if target.dim() != 2 or target.shape[1] != V:
        raise ValueError("target: [rows, V]")
    _need(target, "target", torch.float32, None, dev)
    _need(ell, "ell", torch.int32, (B,), dev)
    if row_offsets is not None:
        _need(row_offsets, "row_offsets", torch.int32, (B + 1,), dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(x, "x", torch.int32, (B, gamma), dev)
    _need(lse_q, "lse_q", torch.float32, (B, gamma), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    if out is None:
        out = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, gamma), dev)
    nbytes = lib.dspark_acceptance_workspace_size(B, gamma, V, r)
    if nbytes == 0:
        raise DSparkError(DSPARK_ERR_ARG, "dspark_acceptance_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    fn = lib.dspark_acceptance if rows is None else lib.dspark_acceptance_rnn
    st = fn(_ptr(target), target.shape[0], _ptr(ell), _ptr(row_offsets),
            _ptr(U), _ptr(W1 if rows is None else rows), _ptr(W2), wdt, _ptr(anchor), _ptr(x), _ptr(lse_q),
            _ptr(temperature), B, gamma, V, r, _ptr(out), _ptr(ws), ws.numel(), _stream_ptr(stream))
    _check(st, "dspark_acceptance" if rows is None else "dspark_acceptance_rnn")
    return out


def dspark_sts_workspace_size(N: int, gamma: int, G: int, n_bins: int) -> int:
    return load_library().dspark_sts_workspace_size(N, gamma, G, n_bins)


def dspark_sts_fit(conf, n_accept, grid, *, ell=None, n_bins: int = 15, ece_grid: bool = False, workspace=None,
                   stream=None) -> dict:
    """Sequential temperature scaling of the confidence head from N observed
    rounds: conf [N, gamma] float32 (raw head, tau = 1), n_accept [N] int32,
    grid [G] float32 temperatures, ell [N] int32 or None (gamma).  Returns
    {"tau" [gamma], "ece" [gamma][, "ece_grid" [gamma, G]]} (device)."""
    torch = _torch()
    lib = load_library()
    dev = conf.device
    N, gamma = conf.shape
    _need(conf, "conf", torch.float32, (N, gamma), dev)
    _need(n_accept, "n_accept", torch.int32, (N,), dev)
    if ell is not None:
        _need(ell, "ell", torch.int32, (N,), dev)
    G = grid.shape[0]
    _need(grid, "grid", torch.float32, (G,), dev)
    out = {"tau": torch.empty(gamma, dtype=torch.float32, device=dev),
           "ece": torch.empty(gamma, dtype=torch.float32, device=dev)}
    if ece_grid:
        out["ece_grid"] = torch.empty((gamma, G), dtype=torch.float32, device=dev)
    nbytes = lib.dspark_sts_workspace_size(N, gamma, G, n_bins)
    if nbytes == 0:
        raise DSparkError(DSPARK_ERR_ARG, "dspark_sts_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    st = lib.dspark_sts_fit(_ptr(conf), _ptr(n_accept), _ptr(ell), N, gamma, _ptr(grid), G, n_bins,
                            _ptr(out["tau"]), _ptr(out["ece"]), _ptr(out.get("ece_grid")), _ptr(ws), ws.numel(),
                            _stream_ptr(stream))
    _check(st, "dspark_sts_fit")
    return out


def dspark_verify_check(workspace, stream=None) -> int:
    """Synchronise and return the device-side input status of the last verify."""
    return load_library().dspark_verify_check(_ptr(workspace), _stream_ptr(stream))


def dspark_schedule(c, sps):
    """Host scheduler.  c [R, gamma] float64 in [0, 1], sps [sps_len] float64.
    Returns (ell [R] int32, theta, tau, B)."""
    lib = load_library()
    c = np.ascontiguousarray(c, dtype=np.float64)
    sps = np.ascontiguousarray(sps, dtype=np.float64)
    if c.ndim != 2:
        raise ValueError("c: [R, gamma]")
    R, gamma = c.shape
    ell = np.zeros(R, np.int32)
    theta = ctypes.c_double()
    tau = ctypes.c_double()
    Bo = ctypes.c_int32()
    st = lib.dspark_schedule(c.ctypes.data_as(_f64p), R, gamma, sps.ctypes.data_as(_f64p), len(sps),
                             ell.ctypes.data_as(_i32p), ctypes.byref(theta), ctypes.byref(tau), ctypes.byref(Bo))
    _check(st, "dspark_schedule")
    return ell, theta.value, tau.value, Bo.value


def dspark_history_capacity(B_hist, R_hist, R: int, gamma: int) -> int:
    """Capacity of the current step from the previous steps' (B, R)."""
    lib = load_library()
    Bh = np.ascontiguousarray(B_hist, dtype=np.int32)
    Rh = np.ascontiguousarray(R_hist, dtype=np.int32)
    cap = ctypes.c_int64()
    st = lib.dspark_history_capacity(Bh.ctypes.data_as(_i32p), Rh.ctypes.data_as(_i32p), len(Bh), R, gamma,
                                     ctypes.byref(cap))
    _check(st, "dspark_history_capacity")
    return cap.value


def dspark_schedule_capacity(c, capacity: int):
    """Fixed-capacity scheduling.  c [R, gamma] float64 in [0, 1].  Returns
    (ell [R] int32, tau, B)."""
    lib = load_library()
    c = np.ascontiguousarray(c, dtype=np.float64)
    if c.ndim != 2:
        raise ValueError("c: [R, gamma]")
    R, gamma = c.shape
    ell = np.zeros(R, np.int32)
    tau = ctypes.c_double()
    Bo = ctypes.c_int32()
    st = lib.dspark_schedule_capacity(c.ctypes.data_as(_f64p), R, gamma, int(capacity), ell.ctypes.data_as(_i32p),
                                      ctypes.byref(tau), ctypes.byref(Bo))
    _check(st, "dspark_schedule_capacity")
    return ell, tau.value, Bo.value


def dspark_debug_random_words(seed, round_id, stream_id, k, req, v0, n, device="cuda", stream=None):
    torch = _torch()
    out = torch.empty(n, dtype=torch.int32, device=device)
    st = load_library().dspark_debug_random_words(int(seed), int(round_id), stream_id, k, req, v0, n,
                                                  _ptr(out), _stream_ptr(stream))
    _check(st, "dspark_debug_random_words")
    return out


def dspark_debug_gumbel(words, stream=None):
    torch = _torch()
    _need(words, "words", torch.int32, None, words.device)
    out = torch.empty(words.numel(), dtype=torch.float32, device=words.device)
    st = load_library().dspark_debug_gumbel(_ptr(words), words.numel(), _ptr(out), _stream_ptr(stream))
    _check(st, "dspark_debug_gumbel")
    return out


def dspark_debug_bias_gemm(W1, W2, idx, *, out=None, workspace=None, stream=None) -> dict:
    """The Markov-bias product alone: rowmax[b] = max_v W1[idx[b]] . W2[v], with
    the draft step's tiling and no sampling.  Returns {"rowmax", "workspace"}."""
    torch = _torch()
    lib = load_library()
    dev = W1.device
    V, r = W1.shape
    wdt = _weights(W1, W2, dev)
    B = idx.numel()
    _need(idx, "idx", torch.int32, (B,), dev)
    if out is None:
        out = {"rowmax": torch.empty(B, dtype=torch.float32, device=dev)}
    nbytes = lib.dspark_draft_workspace_size(B, 1, V, r)
    if nbytes == 0:
        raise DSparkError(DSPARK_ERR_ARG, "dspark_draft_workspace_size")
    ws = _workspace(nbytes, dev, workspace if workspace is not None else out.get("workspace"))
    out["workspace"] = ws
    st = lib.dspark_debug_bias_gemm(_ptr(W1), _ptr(W2), wdt, _ptr(idx), B, V, r, _ptr(out["rowmax"]),
                                    _ptr(ws), ws.numel(), _stream_ptr(stream))
    _check(st, "dspark_debug_bias_gemm")
    return out


def dspark_profile_enable(enable: bool = True):
    _check(load_library().dspark_profile_enable(1 if enable else 0), "dspark_profile_enable")


def dspark_profile_collect():
    _check(load_library().dspark_profile_collect(), "dspark_profile_collect")


def dspark_profile_reset():
    _check(load_library().dspark_profile_reset(), "dspark_profile_reset")


def dspark_profile_read() -> dict:
    """{kernel name: (launches, total milliseconds)} accumulated so far."""
    lib = load_library()
    out = {}
    for i in range(lib.dspark_profile_count()):
        name = ctypes.c_char_p()
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(lib.dspark_profile_get(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)),
               "dspark_profile_get")
        out[name.value.decode()] = (n.value, ms.value)
    return out
