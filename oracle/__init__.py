"""ctypes wrapper around the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.  It takes
numpy arrays, hands raw pointers to the C code and returns numpy arrays.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    lib.orc_philox4x32_10.restype = None
    lib.orc_u01.argtypes = [ctypes.c_uint32]
    lib.orc_u01.restype = ctypes.c_double
    lib.orc_random_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.orc_random_word.restype = ctypes.c_uint32
    lib.orc_draft.argtypes = [_f32p, _f32p, _f32p, _i32p, _f32p, _i32p,
                              ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.c_uint64, ctypes.c_uint64,
                              _i32p, _f64p, _f64p, _f64p]
    lib.orc_draft.restype = ctypes.c_int
    lib.orc_verify.argtypes = [_f32p, _i32p, _i32p, _f32p, _f32p, _f32p, _f32p, _i32p, _i32p, _f32p, _i32p,
                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_uint64, ctypes.c_uint64,
                               _i32p, _i32p, _f64p, _f64p, _f64p, _f64p]
    lib.orc_verify.restype = ctypes.c_int
    lib.orc_confidence.argtypes = [_f32p, _f32p, _f32p, _i32p, _i32p, _f32p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p, _f64p]
    lib.orc_confidence.restype = ctypes.c_int
    lib.orc_acceptance.argtypes = [_f32p, _i32p, _i32p, _f32p, _f32p, _f32p, _f32p, _i32p, _i32p, _f32p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p]
    lib.orc_acceptance.restype = ctypes.c_int
    lib.orc_bf16_round.argtypes = [ctypes.c_double]
    lib.orc_bf16_round.restype = ctypes.c_double
    lib.orc_draft_rnn.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _i32p, _f32p, _i32p,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_uint64, ctypes.c_uint64,
                                  _i32p, _f64p, _f64p, _f64p, _f64p, _f64p]
    lib.orc_draft_rnn.restype = ctypes.c_int
    lib.orc_sts_fit.argtypes = [_f32p, _i32p, _i32p, ctypes.c_int, ctypes.c_int, _f32p, ctypes.c_int,
                                ctypes.c_int, _f64p, _f64p, _f64p]
    lib.orc_sts_fit.restype = ctypes.c_int
    lib.orc_history_capacity.argtypes = [_i32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.orc_history_capacity.restype = ctypes.c_int64
    lib.orc_schedule_capacity.argtypes = [_f64p, ctypes.c_int, ctypes.c_int, ctypes.c_int64, _i32p, _f64p, _i32p]
    lib.orc_schedule_capacity.restype = ctypes.c_int
    lib.orc_schedule.argtypes = [_f64p, ctypes.c_int, ctypes.c_int, _f64p, ctypes.c_int,
                                 _i32p, _f64p, _f64p, _i32p]
    lib.orc_schedule.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def philox4x32_10(counter, key):
    """Raw Philox4x32-10 block: 4 counter words, 2 key words -> 4 words."""
    lib = _load()
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.orc_philox4x32_10(_ptr(c, ctypes.c_uint32), _ptr(k, ctypes.c_uint32), _ptr(out, ctypes.c_uint32))
    return out


def u01(word):
    return _load().orc_u01(int(word))


def random_word(seed, round_id, stream, k, req, v):
    return _load().orc_random_word(seed, round_id, stream, k, req, v)


def draft(U, W1, W2, anchor, temperature, seed, round_id, req_ids=None):
    """Markov-head draft sampling.  U [B, gamma, V], W1/W2 [V, r] (float32
    values; bf16 weights pass their exact float32 value).  Returns a dict of
    x [B, gamma] int32 and lse, qx, margin [B, gamma] float64."""
    lib = _load()
    U = _f32(U)
    W1 = _f32(W1)
    W2 = _f32(W2)
    anchor = _i32(anchor)
    temperature = _f32(temperature)
    B, gamma, V = U.shape
    r = W1.shape[1]
    assert W1.shape == (V, r) and W2.shape == (V, r)
    rid = None if req_ids is None else _i32(req_ids)
    x = np.zeros((B, gamma), np.int32)
    lse = np.zeros((B, gamma), np.float64)
    qx = np.zeros((B, gamma), np.float64)
    margin = np.zeros((B, gamma), np.float64)
    st = lib.orc_draft(_ptr(U, ctypes.c_float), _ptr(W1, ctypes.c_float), _ptr(W2, ctypes.c_float),
                       _ptr(anchor, ctypes.c_int32), _ptr(temperature, ctypes.c_float),
                       _ptr(rid, ctypes.c_int32), B, gamma, V, r, seed, round_id,
                       _ptr(x, ctypes.c_int32), _ptr(lse, ctypes.c_double),
                       _ptr(qx, ctypes.c_double), _ptr(margin, ctypes.c_double))
    if st != 0:
        raise ValueError("orc_draft: bad arguments")
    return {"x": x, "lse": lse, "qx": qx, "margin": margin}


def bf16_round(x):
    """x rounded to the nearest bfloat16 value, ties to even (from double)."""
    return _load().orc_bf16_round(float(x))


def draft_rnn(U, W1, W2, Wgco, h, anchor, temperature, seed, round_id, req_ids=None):
    """Draft sampling with the RNN head.  U [B, gamma, V], W1/W2 [V, r],
    Wgco [3r, 2r + d], h [B, gamma, d] (float32 values).  Returns the dict of
    draft() plus the final state [B, r] and the head rows e [B, gamma, r]
    (bfloat16 values) the W2 product used, both float64."""
    lib = _load()
    U = _f32(U)
    W1 = _f32(W1)
    W2 = _f32(W2)
    Wgco = _f32(Wgco)
    h = _f32(h)
    anchor = _i32(anchor)
    temperature = _f32(temperature)
    B, gamma, V = U.shape
    r = W1.shape[1]
    d = h.shape[2]
    assert Wgco.shape == (3 * r, 2 * r + d) and h.shape[:2] == (B, gamma)
    rid = None if req_ids is None else _i32(req_ids)
    x = np.zeros((B, gamma), np.int32)
    lse = np.zeros((B, gamma), np.float64)
    qx = np.zeros((B, gamma), np.float64)
    margin = np.zeros((B, gamma), np.float64)
    state = np.zeros((B, r), np.float64)
    e = np.zeros((B, gamma, r), np.float64)
    st = lib.orc_draft_rnn(_ptr(U, ctypes.c_float), _ptr(W1, ctypes.c_float), _ptr(W2, ctypes.c_float),
                           _ptr(Wgco, ctypes.c_float), _ptr(h, ctypes.c_float) if d > 0 else None,
                           _ptr(anchor, ctypes.c_int32), _ptr(temperature, ctypes.c_float),
                           _ptr(rid, ctypes.c_int32), B, gamma, V, r, d, seed, round_id,
                           _ptr(x, ctypes.c_int32), _ptr(lse, ctypes.c_double),
                           _ptr(qx, ctypes.c_double), _ptr(margin, ctypes.c_double),
                           _ptr(state, ctypes.c_double), _ptr(e, ctypes.c_double))
    if st != 0:
        raise ValueError("orc_draft_rnn: bad arguments")
    return {"x": x, "lse": lse, "qx": qx, "margin": margin, "state": state, "e": e}


def verify(target, ell, U, W1, W2, anchor, x, temperature, seed, round_id,
           req_ids=None, row_offsets=None, head_rows=None):
    """Exact rejection-sampling verification against packed target rows
    [sum(1 + ell), V].  head_rows [B, gamma, r]: the rows the head fed the W2
    product (the RNN head's e_k); None: the Markov head's W1[x_{k-1}].
    Returns n [B], tokens [B, gamma+1], diag [B, gamma+1, 2], resid [B],
    accept_margin [B, gamma], pick_margin [B]."""
    lib = _load()
    target = _f32(target)
    U = _f32(U)
    W1 = _f32(W1)
    W2 = _f32(W2)
    ell = _i32(ell)
    anchor = _i32(anchor)
    x = _i32(x)
    temperature = _f32(temperature)
    B, gamma, V = U.shape
    r = W1.shape[1]
    rid = None if req_ids is None else _i32(req_ids)
    off = None if row_offsets is None else _i32(row_offsets)
    E = None if head_rows is None else _f32(head_rows)
    n = np.zeros(B, np.int32)
    tokens = np.zeros((B, gamma + 1), np.int32)
    diag = np.zeros((B, gamma + 1, 2), np.float64)
    resid = np.zeros(B, np.float64)
    am = np.zeros((B, gamma), np.float64)
    pm = np.zeros(B, np.float64)
    st = lib.orc_verify(_ptr(target, ctypes.c_float), _ptr(off, ctypes.c_int32), _ptr(ell, ctypes.c_int32),
                        _ptr(U, ctypes.c_float), _ptr(W1, ctypes.c_float), _ptr(W2, ctypes.c_float),
                        _ptr(E, ctypes.c_float), _ptr(anchor, ctypes.c_int32), _ptr(x, ctypes.c_int32),
                        _ptr(temperature, ctypes.c_float), _ptr(rid, ctypes.c_int32),
                        B, gamma, V, r, seed, round_id,
                        _ptr(n, ctypes.c_int32), _ptr(tokens, ctypes.c_int32),
                        _ptr(diag, ctypes.c_double), _ptr(resid, ctypes.c_double),
                        _ptr(am, ctypes.c_double), _ptr(pm, ctypes.c_double))
    if st != 0:
        raise ValueError("orc_verify: bad arguments")
    return {"n": n, "tokens": tokens, "diag": diag, "resid": resid,
            "accept_margin": am, "pick_margin": pm}


def confidence(h, w, W1, anchor, x, tau=None):
    """Confidence head and prefix survival.  h [B, gamma, d], w [d + r],
    W1 [V, r], anchor [B], drafts x [B, gamma].  Returns (c, a), both
    [B, gamma] float64.  tau [gamma]: temperatures of the head's logits."""
    lib = _load()
    h = _f32(h)
    w = _f32(w)
    W1 = _f32(W1)
    anchor = _i32(anchor)
    x = _i32(x)
    B, gamma, d = h.shape
    r = W1.shape[1]
    assert w.shape == (d + r,) and x.shape == (B, gamma)
    t = None if tau is None else _f32(tau)
    c = np.zeros((B, gamma), np.float64)
    a = np.zeros((B, gamma), np.float64)
    st = lib.orc_confidence(_ptr(h, ctypes.c_float), _ptr(w, ctypes.c_float), _ptr(W1, ctypes.c_float),
                            _ptr(anchor, ctypes.c_int32), _ptr(x, ctypes.c_int32), _ptr(t, ctypes.c_float),
                            B, gamma, d, r,
                            _ptr(c, ctypes.c_double), _ptr(a, ctypes.c_double))
    if st != 0:
        raise ValueError("orc_confidence: bad arguments")
    return c, a


def acceptance(target, ell, U, W1, W2, anchor, x, temperature, row_offsets=None, head_rows=None):
    """Per-position acceptance probability alpha_k = sum_v min(p_k, q_k) for
    k <= ell_b over packed target rows [sum(1 + ell), V]; NaN past ell_b.
    Returns alpha [B, gamma] float64."""
    lib = _load()
    target = _f32(target)
    U = _f32(U)
    W1 = _f32(W1)
    W2 = _f32(W2)
    ell = _i32(ell)
    anchor = _i32(anchor)
    x = _i32(x)
    temperature = _f32(temperature)
    B, gamma, V = U.shape
    r = W1.shape[1]
    off = None if row_offsets is None else _i32(row_offsets)
    E = None if head_rows is None else _f32(head_rows)
    alpha = np.zeros((B, gamma), np.float64)
    st = lib.orc_acceptance(_ptr(target, ctypes.c_float), _ptr(off, ctypes.c_int32), _ptr(ell, ctypes.c_int32),
                            _ptr(U, ctypes.c_float), _ptr(W1, ctypes.c_float), _ptr(W2, ctypes.c_float),
                            _ptr(E, ctypes.c_float), _ptr(anchor, ctypes.c_int32), _ptr(x, ctypes.c_int32),
                            _ptr(temperature, ctypes.c_float), B, gamma, V, r, _ptr(alpha, ctypes.c_double))
    if st != 0:
        raise ValueError("orc_acceptance: bad arguments")
    return alpha


def sts_fit(c, n, grid, n_bins=15, ell=None):
    """Sequential temperature scaling.  c [N, gamma] confidences, n [N]
    accepted counts, grid [G] temperatures, ell [N] verified lengths (None:
    gamma).  Returns (tau [gamma], ece [gamma], ece_grid [gamma, G])."""
    lib = _load()
    c = _f32(c)
    n = _i32(n)
    grid = _f32(grid)
    N, gamma = c.shape
    L = None if ell is None else _i32(ell)
    tau = np.zeros(gamma, np.float64)
    ece = np.zeros(gamma, np.float64)
    eg = np.zeros((gamma, len(grid)), np.float64)
    st = lib.orc_sts_fit(_ptr(c, ctypes.c_float), _ptr(n, ctypes.c_int32), _ptr(L, ctypes.c_int32), N, gamma,
                         _ptr(grid, ctypes.c_float), len(grid), n_bins, _ptr(tau, ctypes.c_double),
                         _ptr(ece, ctypes.c_double), _ptr(eg, ctypes.c_double))
    if st != 0:
        raise ValueError("orc_sts_fit: bad arguments")
    return tau, ece, eg


def schedule(c, sps):
    """Confidence-scheduled prefix lengths.  c [R, gamma] float64, sps
    [sps_len] float64 (SPS(B) for B = 0..sps_len-1).  Returns
    (ell [R] int32, theta, tau, B)."""
    lib = _load()
    c = np.ascontiguousarray(c, dtype=np.float64)
    sps = np.ascontiguousarray(sps, dtype=np.float64)
    R, gamma = c.shape
    ell = np.zeros(R, np.int32)
    theta = ctypes.c_double()
    tau = ctypes.c_double()
    Bo = ctypes.c_int32()
    st = lib.orc_schedule(_ptr(c, ctypes.c_double), R, gamma, _ptr(sps, ctypes.c_double), len(sps),
                          _ptr(ell, ctypes.c_int32), ctypes.byref(theta), ctypes.byref(tau), ctypes.byref(Bo))
    if st != 0:
        raise ValueError("orc_schedule: bad arguments")
    return ell, theta.value, tau.value, Bo.value


def history_capacity(B_hist, R_hist, R, gamma):
    """Capacity of the current step from the previous steps' (B, R)."""
    B_hist = _i32(B_hist)
    R_hist = _i32(R_hist)
    return int(_load().orc_history_capacity(_ptr(B_hist, ctypes.c_int32), _ptr(R_hist, ctypes.c_int32),
                                            len(B_hist), R, gamma))


def schedule_capacity(c, capacity):
    """Lengths for a fixed capacity: (ell [R] int32, tau, B)."""
    lib = _load()
    c = np.ascontiguousarray(c, dtype=np.float64)
    R, gamma = c.shape
    ell = np.zeros(R, np.int32)
    tau = ctypes.c_double()
    Bo = ctypes.c_int32()
    st = lib.orc_schedule_capacity(_ptr(c, ctypes.c_double), R, gamma, int(capacity), _ptr(ell, ctypes.c_int32),
                                   ctypes.byref(tau), ctypes.byref(Bo))
    if st != 0:
        raise ValueError("orc_schedule_capacity: bad arguments")
    return ell, tau.value, Bo.value
