"""Seeded synthetic inputs for one draft-and-verify round.

This module holds random draws and data layout only -- none of the method's
arithmetic.  Both the HIP library's tests/benchmark and the CPU oracle are
fed from here, so the two sides always see the same bits.

Recipe (every stream is its own numpy PCG64 generator seeded with a tuple,
so any request's rows can be regenerated on their own):
  W1, W2 [V, r]      ~ N(0, w_std)    seeds (seed, 0) and (seed, 1); bf16
                                      configs round the float32 draw to
                                      bfloat16 with round-to-nearest-even.
  U[b, k] [V]        ~ N(0, u_std)    seed (seed, 2, b, k), k = 1..gamma+1;
                                      row gamma+1 is a phantom position used
                                      only by the bonus target row.
  t[b, k] [V]        = U[b, k] + N(0, sigma_k)   seed (seed, 3, b, k).
  anchor [B]         ~ uniform [0, V)  seed (seed, 4).
  c [B, gamma]       ~ Beta(8, 2)     seed (seed, 5)   (scheduled config).
  temperature [B]    1.0, or 0.0 (greedy) for b % greedy_every == 0.
  RNN head (rnn_head_weights): Wgco [3r, 2r + d] ~ N(0, (2r + d)^-1/2),
                     seed (seed, 9), rounded to bfloat16; it reads the same
                     h as the confidence head.
  Calibration samples (sts_samples): true conditional logits s ~ N(0.8, 1.5)
                     seed (seed, 10); position k survives iff k - 1 did and
                     u < sigmoid(s_k), u ~ U(0, 1) seed (seed, 11); the head
                     reports sigmoid(scale_k s_k) (scale > 1: overconfident).
  Confidence head (confidence_head_inputs; d defaults to 1024):
  h[b, k] [d]        ~ N(1, 1)        seed (seed, 6, b, k)
  w [d + r]          first d ~ N(1.4 / d, 0.5 / d), seed (seed, 7); last r
                     ~ N(0, 0.5 / (r w_std^2)), seed (seed, 8) -- so the head's
                     logit is about N(1.4, 1.5) and c_k averages about 0.7.
The target rows are packed per request: rows k = 1..ell_b + 1 of request b
follow each other, request after request.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["Config", "CONFIGS", "Round", "make_round", "bf16_round", "bf16_bits_to_f32",
           "sps_table_toy", "pack_offsets", "confidence_head_inputs", "rnn_head_weights",
           "sts_samples", "DEFAULT_HIDDEN"]

DEFAULT_HIDDEN = 1024


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    gamma: int
    V: int
    r: int
    wdtype: str  # "bf16" or "f32"
    w_std: float
    u_std: float
    noise_std: float  # constant sigma, unless sigma_ramp is set
    seed: int
    greedy_every: int = 0  # 0: no greedy requests
    sigma_ramp: tuple | None = None  # (first, last) linear over k = 1..gamma
    sigma_bonus: float | None = None  # sigma of the phantom row gamma+1
    scheduled: bool = False

    def sigma(self, k: int) -> float:
        """Noise std of target row k (1-based; k = gamma + 1 is the phantom row)."""
        if self.sigma_ramp is None:
            return self.noise_std
        if k > self.gamma:
            return self.sigma_bonus if self.sigma_bonus is not None else self.sigma_ramp[1]
        a, b = self.sigma_ramp
        return a + (b - a) * (k - 1) / max(1, self.gamma - 1)

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # batch 1, gamma 4, V 1000, rank 16, float32 everywhere
    "tiny": Config("tiny", B=1, gamma=4, V=1000, r=16, wdtype="f32", w_std=0.1,
                   u_std=2.0, noise_std=0.5, seed=0),
    # DSpark-5 style: batch 32, gamma 5, V 151936, rank 256, bf16 weights
    "dspark5": Config("dspark5", B=32, gamma=5, V=151936, r=256, wdtype="bf16", w_std=0.02,
                      u_std=3.0, noise_std=1.0, seed=1),
    # Large batch: batch 256, gamma 5, V 129280, rank 256, 10% greedy requests
    "large": Config("large", B=256, gamma=5, V=129280, r=256, wdtype="bf16", w_std=0.02,
                    u_std=3.0, noise_std=1.0, seed=2, greedy_every=10),
    # Long block: batch 64, gamma 16, sigma_k 0.5 -> 2.0 over positions
    "long": Config("long", B=64, gamma=16, V=151936, r=256, wdtype="bf16", w_std=0.02,
                   u_std=3.0, noise_std=1.0, seed=3, sigma_ramp=(0.5, 2.0), sigma_bonus=2.0),
    # Scheduled ragged verify: batch 1024, confidences ~ Beta(8, 2)
    "sched": Config("sched", B=1024, gamma=5, V=129280, r=256, wdtype="bf16", w_std=0.02,
                    u_std=3.0, noise_std=1.0, seed=4, scheduled=True),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seq, n, std) -> np.ndarray:
    g = np.random.default_rng(seq)
    a = g.standard_normal(n, dtype=np.float32)
    a *= np.float32(std)
    return a


def pack_offsets(ell: np.ndarray) -> np.ndarray:
    """Exclusive scan of (1 + ell): first packed target row of each request, plus the total."""
    ell = np.asarray(ell, dtype=np.int64)
    off = np.zeros(len(ell) + 1, dtype=np.int64)
    np.cumsum(1 + ell, out=off[1:])
    return off.astype(np.int32)


def sps_table_toy(rho: float, n: int) -> np.ndarray:
    """SPS(B) = 1000 / T(B) for the interactive page's teaching cost curve
    T(B) = 20 + (0.05 + 1.15 rho) B + (0.002 + 0.10 rho) B^2 milliseconds,
    tabulated for B = 0..n-1."""
    B = np.arange(n, dtype=np.float64)
    T = 20.0 + (0.05 + 1.15 * rho) * B + (0.002 + 0.10 * rho) * B * B
    return 1000.0 / T


@dataclasses.dataclass
class Round:
    cfg: Config
    W1_bits: np.ndarray | None  # [V, r] uint16 (bf16 configs)
    W2_bits: np.ndarray | None
    W1: np.ndarray  # [V, r] float32 values (exact bf16 values for bf16 configs)
    W2: np.ndarray
    U: np.ndarray  # [B, gamma, V] float32
    anchor: np.ndarray  # [B] int32
    temperature: np.ndarray  # [B] float32
    c: np.ndarray | None  # [B, gamma] float64
    seed: int
    requests: list  # global request index of each local row

    @property
    def B(self):
        return len(self.requests)

    def weights_device_layout(self):
        """(W1, W2) arrays in the element type the library takes."""
        if self.cfg.wdtype == "bf16":
            return self.W1_bits, self.W2_bits
        return self.W1, self.W2

    def target_row(self, i: int, k: int) -> np.ndarray:
        """Target logits for local request row i, position k (1-based, up to gamma+1)."""
        cfg = self.cfg
        b = self.requests[i]
        if k <= cfg.gamma:
            u = self.U[i, k - 1]
        else:
            u = _normal((cfg.seed, 2, b, k), cfg.V, cfg.u_std)
        return u + _normal((cfg.seed, 3, b, k), cfg.V, cfg.sigma(k))

    def target_packed(self, ell: np.ndarray) -> np.ndarray:
        """Packed target rows [sum(1 + ell), V], request after request
        (ell indexed by local request row)."""
        jobs = [(i, k) for i in range(self.B) for k in range(1, int(ell[i]) + 2)]
        out = np.empty((len(jobs), self.cfg.V), dtype=np.float32)

        def fill(i):
            b, k = jobs[i]
            out[i] = self.target_row(b, k)

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(jobs))))
        return out


def make_round(cfg: Config, requests=None) -> Round:
    """Generate the weights, base logits, anchors, temperatures (and
    confidences for the scheduled config) of ``cfg``.  ``requests`` limits U
    to those request rows (in that order); W1/W2 are always full."""
    V, r, gamma = cfg.V, cfg.r, cfg.gamma
    with ThreadPoolExecutor(2) as ex:
        f1 = ex.submit(_normal, (cfg.seed, 0), V * r, cfg.w_std)
        f2 = ex.submit(_normal, (cfg.seed, 1), V * r, cfg.w_std)
        w1, w2 = f1.result().reshape(V, r), f2.result().reshape(V, r)
    if cfg.wdtype == "bf16":
        W1_bits, W2_bits = bf16_round(w1), bf16_round(w2)
        W1, W2 = bf16_bits_to_f32(W1_bits), bf16_bits_to_f32(W2_bits)
    else:
        W1_bits = W2_bits = None
        W1, W2 = w1, w2
    reqs = list(range(cfg.B)) if requests is None else list(requests)
    U = np.empty((len(reqs), gamma, V), dtype=np.float32)

    def fill(i):
        b = reqs[i // gamma]
        k = i % gamma + 1
        U[i // gamma, k - 1] = _normal((cfg.seed, 2, b, k), V, cfg.u_std)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(reqs) * gamma)))
    anchor_all = np.random.default_rng((cfg.seed, 4)).integers(0, V, size=cfg.B).astype(np.int32)
    temp_all = np.ones(cfg.B, dtype=np.float32)
    if cfg.greedy_every:
        temp_all[::cfg.greedy_every] = 0.0
    c = None
    if cfg.scheduled:
        c_all = np.random.default_rng((cfg.seed, 5)).beta(8.0, 2.0, size=(cfg.B, gamma))
        c = c_all[reqs]
    return Round(cfg=cfg, W1_bits=W1_bits, W2_bits=W2_bits, W1=W1, W2=W2, U=U,
                 anchor=anchor_all[reqs], temperature=temp_all[reqs], c=c, seed=cfg.seed,
                 requests=reqs)


def confidence_head_inputs(cfg: Config, d: int = DEFAULT_HIDDEN, requests=None):
    """(h [B, gamma, d], w [d + r]) float32 for the confidence head of ``cfg``
    (``requests`` selects request rows, in that order)."""
    reqs = list(range(cfg.B)) if requests is None else list(requests)
    h = np.empty((len(reqs), cfg.gamma, d), dtype=np.float32)
    for i, b in enumerate(reqs):
        for k in range(1, cfg.gamma + 1):
            h[i, k - 1] = _normal((cfg.seed, 6, b, k), d, 1.0) + np.float32(1.0)
    w = np.empty(d + cfg.r, dtype=np.float32)
    if d > 0:
        w[:d] = _normal((cfg.seed, 7), d, np.sqrt(0.5 / d)) + np.float32(1.4 / d)
    w[d:] = _normal((cfg.seed, 8), cfg.r, np.sqrt(0.5 / (cfg.r * cfg.w_std ** 2)))
    return h, w


def rnn_head_weights(cfg: Config, d: int = DEFAULT_HIDDEN):
    """(Wgco bfloat16 bits [3r, 2r + d] uint16, their float32 values) for the
    RNN head of ``cfg``."""
    K = 2 * cfg.r + d
    w = _normal((cfg.seed, 9), 3 * cfg.r * K, 1.0 / np.sqrt(K)).reshape(3 * cfg.r, K)
    bits = bf16_round(w)
    return bits, bf16_bits_to_f32(bits)


def sts_samples(N: int, scales, seed: int):
    """(c [N, gamma] float32, n [N] int32): N synthetic rounds whose reported
    confidences are miscalibrated by known logit scales (recipe above)."""
    gamma = len(scales)
    s = np.random.default_rng((seed, 10)).normal(0.8, 1.5, (N, gamma))
    u = np.random.default_rng((seed, 11)).uniform(size=(N, gamma))
    accept = u < 1.0 / (1.0 + np.exp(-s))
    n = np.argmin(np.concatenate([accept, np.zeros((N, 1), bool)], axis=1), axis=1).astype(np.int32)
    c = (1.0 / (1.0 + np.exp(-np.asarray(scales, np.float64) * s))).astype(np.float32)
    return c, n
