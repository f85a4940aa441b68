"""Synthetic workloads for one UA layer: decode and prefill configurations.

The shapes follow a 1B Llama3-style layer (hidden 2048, 32 query / 8 KV
heads, head dim 64) and a 3B-style layer (hidden 3072, 24 / 8 heads, head
dim 128).  Cache statistics stand in for the paper's RULER / LongBench-E
evaluations (paperlayer.ai summary, sections 5.1-5.4; ai4snews page): nominal
contexts of 4096 (training length) and 16384 (the 16k evaluation), mean
compression 10x and 25x, maximum 114x, thresholds p = 0.05 and 0.15.  No
dataset is read: everything is drawn from seeded numpy generators (PCG64).

Draw order for a configuration and seed: SeedSequence(seed).spawn(3) gives
independent streams for (weights, initial cache, per-step inputs); per-step
inputs of step i come from the step stream's i-th spawned child, so any step
can be drawn on its own.

Values are returned as float32 arrays.  In bf16 configurations every value the
device reads as bf16 (q, k, v, x, weights, cached K and V) is already rounded
to bf16, so the same numbers reach the oracle and the GPU.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np


# ---------------------------------------------------------------------------
# bf16 helpers (torch's round-to-nearest-even conversion)
# ---------------------------------------------------------------------------
def bf16_exact(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 and return them as float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bf16-exact float32 values (upper halves)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class LayerConfig:
    name: str
    B: int
    H_q: int
    H_kv: int
    d: int
    D: int
    r: int = 16
    bf16: bool = True
    mode: str = "decode"  # "decode" or "prefill"
    steps: int = 0  # decode steps
    p: float = 0.15
    b_dec: str = "const-2"  # "const-2" or "uniform-4-0"
    # initial cache (decode)
    len_kind: str = "empty"  # "empty", "lognormal", "ragged"
    len_mean: float = 0.0
    len_min: int = 16
    len_max: int = 0
    nominal: int = 0  # starting position for decode
    lam_p0: float = 0.15  # initial Lambda ~ U[log p0, 0]
    nom_lo: int = 0  # ragged: nominal context range
    nom_hi: int = 0
    rho_lo: float = 2.0  # ragged: per-head compression range
    rho_hi: float = 114.0
    # prefill
    n_total: int = 0
    chunk: int = 0
    w_var: float = 1.0 / 64.0  # variance of W_dec, W_dn, W_up entries
    q_scale: float = 1.0  # queries are N(0, q_scale^2); a power of two keeps bf16 draws exact

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv


CONFIGS: Dict[str, LayerConfig] = {
    # tiny fp32 decode from an empty cache; the oracle finishes in seconds
    "tiny-decode-f32": LayerConfig(
        name="tiny-decode-f32", B=1, H_q=1, H_kv=1, d=64, D=64, bf16=False, steps=256, p=0.15, nominal=0
    ),
    # 1B-shape decode on a pre-populated pruned cache, nominal 4096, ~10x
    "1b-decode": LayerConfig(
        name="1b-decode", B=8, H_q=32, H_kv=8, d=64, D=2048, steps=512, p=0.15, len_kind="lognormal",
        len_mean=4096 / 10, len_min=16, len_max=4096, nominal=4096, lam_p0=0.15
    ),
    # 1B-shape chunked prefill, 16384 tokens in 1024-token calls, then eviction at p = 0.05
    "1b-prefill": LayerConfig(
        name="1b-prefill", B=2, H_q=32, H_kv=8, d=64, D=2048, mode="prefill", p=0.05, b_dec="uniform-4-0",
        n_total=16384, chunk=1024
    ),
    # 3B-shape long-context decode, nominal 16384, ~25x (at least 1/114 kept)
    "3b-decode": LayerConfig(
        name="3b-decode", B=16, H_q=24, H_kv=8, d=128, D=3072, steps=256, p=0.15, len_kind="lognormal",
        len_mean=16384 / 25, len_min=math.ceil(16384 / 114), len_max=16384, nominal=16384, lam_p0=0.15
    ),
    # ragged stress: B = 64, nominal 1k..32k, per-head compression 2..114
    "ragged-decode": LayerConfig(
        name="ragged-decode", B=64, H_q=32, H_kv=8, d=64, D=2048, steps=128, p=0.05, b_dec="uniform-4-0",
        len_kind="ragged", nom_lo=1024, nom_hi=32768, lam_p0=0.05
    ),
}


def config(name: str, **overrides) -> LayerConfig:
    return replace(CONFIGS[name], **overrides)


# ---------------------------------------------------------------------------
# containers
# ---------------------------------------------------------------------------
@dataclass
class Weights:
    W_dec: np.ndarray  # [D, 3*H_kv]   (bf16-exact in bf16 configs)
    b_dec: np.ndarray  # [3*H_kv] float32
    W_dn: np.ndarray  # [D, r]
    W_up: np.ndarray  # [r, H_q*d]
    b_up: np.ndarray  # [H_q*d] float32 (zeros)


@dataclass
class CacheInit:
    """Initial cache in the slot layout the library uses.

    Segment s = b*H_kv + h owns slots [seg_off[s], seg_off[s] + seg_cap[s]);
    its first seg_len[s] slots hold live entries in insertion order.
    """

    K: np.ndarray  # [slots, d] float32 (bf16-exact in bf16 configs)
    V: np.ndarray  # [slots, d]
    lam: np.ndarray  # [slots] float32
    lk: np.ndarray  # [slots] float32
    seg_off: np.ndarray  # [S] int64
    seg_len: np.ndarray  # [S] int32
    seg_cap: np.ndarray  # [S] int32
    next_pos: np.ndarray  # [B] int32

    @property
    def slots(self) -> int:
        return int(self.K.shape[0])


@dataclass
class StepInputs:
    q: np.ndarray  # [B, n, H_q, d]
    k: np.ndarray  # [B, n, H_kv, d]
    v: np.ndarray  # [B, n, H_kv, d]
    x: np.ndarray  # [B, n, D]


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------
def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    w, c, s = ss.spawn(3)
    return w, c, s


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_weights(cfg: LayerConfig, seed: int = 0) -> Weights:
    rng = np.random.Generator(np.random.PCG64(_streams(seed)[0]))
    std = math.sqrt(cfg.w_var)
    W_dec = _normal(rng, (cfg.D, 3 * cfg.H_kv), std)
    W_dn = _normal(rng, (cfg.D, cfg.r), std)
    W_up = _normal(rng, (cfg.r, cfg.H_q * cfg.d), std)
    if cfg.b_dec == "const-2":
        b_dec = np.full(3 * cfg.H_kv, -2.0, np.float32)
    else:
        b_dec = rng.uniform(-4.0, 0.0, 3 * cfg.H_kv).astype(np.float32)
    if cfg.bf16:
        W_dec, W_dn, W_up = bf16_exact(W_dec), bf16_exact(W_dn), bf16_exact(W_up)
    return Weights(W_dec=W_dec, b_dec=b_dec, W_dn=W_dn, W_up=W_up, b_up=np.zeros(cfg.H_q * cfg.d, np.float32))


def make_layout(lengths: np.ndarray, extra: int, align: int = 16):
    """Segment offsets/capacities: capacity = len + extra rounded up to ``align``."""
    lengths = np.asarray(lengths, np.int64)
    cap = ((lengths + extra + align - 1) // align) * align
    cap = np.maximum(cap, align)
    off = np.zeros_like(cap)
    off[1:] = np.cumsum(cap)[:-1]
    return off.astype(np.int64), cap.astype(np.int32), int(cap.sum())


def _initial_lengths(cfg: LayerConfig, rng: np.random.Generator):
    S = cfg.B * cfg.H_kv
    if cfg.len_kind == "empty":
        return np.zeros(S, np.int64), np.full(cfg.B, cfg.nominal, np.int64)
    if cfg.len_kind == "lognormal":
        mu = math.log(cfg.len_mean) - 0.5  # mean of LogNormal(mu, 1) = len_mean
        raw = rng.lognormal(mu, 1.0, S)
        n = np.clip(np.rint(raw), cfg.len_min, cfg.len_max).astype(np.int64)
        return n, np.full(cfg.B, cfg.nominal, np.int64)
    if cfg.len_kind == "ragged":
        nom = rng.integers(cfg.nom_lo, cfg.nom_hi + 1, cfg.B)
        rho = rng.uniform(cfg.rho_lo, cfg.rho_hi, S)
        n = np.rint(np.repeat(nom, cfg.H_kv) / rho).astype(np.int64)
        n = np.clip(n, 16, np.repeat(nom, cfg.H_kv))
        return n, nom.astype(np.int64)
    raise ValueError(cfg.len_kind)


def make_cache(cfg: LayerConfig, weights: Weights, seed: int = 0, extra: Optional[int] = None) -> CacheInit:
    """Pre-populated pruned cache (or an empty one) with room for ``extra`` appends.

    Stored keys are normalised N(0, I) vectors rounded to the cache dtype and
    taken as already rotated; values are N(0, 1); Lambda ~ U[log p0, 0]; the
    stored key gate is a draw of log sigmoid(z) with z ~ N(b_k, ||w_k||^2),
    the law of x.w_k + b_k for x ~ N(0, I).
    """
    rng = np.random.Generator(np.random.PCG64(_streams(seed)[1]))
    lengths, nominal = _initial_lengths(cfg, rng)
    if extra is None:
        extra = cfg.steps if cfg.mode == "decode" else cfg.n_total
    off, cap, slots = make_layout(lengths, extra)
    S = cfg.B * cfg.H_kv
    K = np.zeros((slots, cfg.d), np.float32)
    V = np.zeros((slots, cfg.d), np.float32)
    lam = np.zeros(slots, np.float32)
    lk = np.zeros(slots, np.float32)
    wk_norm = np.linalg.norm(weights.W_dec[:, cfg.H_kv : 2 * cfg.H_kv].astype(np.float64), axis=0)
    for s in range(S):
        n = int(lengths[s])
        if n == 0:
            continue
        h = s % cfg.H_kv
        kk = rng.standard_normal((n, cfg.d))
        kk /= np.linalg.norm(kk, axis=1, keepdims=True)
        K[off[s] : off[s] + n] = kk.astype(np.float32)
        V[off[s] : off[s] + n] = rng.standard_normal((n, cfg.d), dtype=np.float32)
        lam[off[s] : off[s] + n] = rng.uniform(math.log(cfg.lam_p0), 0.0, n).astype(np.float32)
        z = rng.normal(float(weights.b_dec[cfg.H_kv + h]), float(wk_norm[h]), n)
        lk[off[s] : off[s] + n] = (-np.logaddexp(0.0, -z)).astype(np.float32)
    if cfg.bf16:
        K, V = bf16_exact(K), bf16_exact(V)
    return CacheInit(K=K, V=V, lam=lam, lk=lk, seg_off=off, seg_len=lengths.astype(np.int32), seg_cap=cap,
                     next_pos=nominal.astype(np.int32))


def make_step_inputs(cfg: LayerConfig, step: int, n: int = 1, seed: int = 0) -> StepInputs:
    """Inputs of decode step ``step`` (n = 1) or prefill call ``step`` (n tokens)."""
    ss = _streams(seed)[2]
    child = np.random.SeedSequence(entropy=ss.entropy, spawn_key=ss.spawn_key + (step,))
    rng = np.random.Generator(np.random.PCG64(child))
    q = _normal(rng, (cfg.B, n, cfg.H_q, cfg.d)) * cfg.q_scale
    k = _normal(rng, (cfg.B, n, cfg.H_kv, cfg.d))
    v = _normal(rng, (cfg.B, n, cfg.H_kv, cfg.d))
    x = _normal(rng, (cfg.B, n, cfg.D))
    if cfg.bf16:
        q, k, v, x = bf16_exact(q), bf16_exact(k), bf16_exact(v), bf16_exact(x)
    return StepInputs(q=q, k=k, v=v, x=x)


# ---------------------------------------------------------------------------
# inputs of the attention backward (one training chunk per sequence)
# ---------------------------------------------------------------------------
@dataclass
class GradInputs:
    q: np.ndarray  # rotated queries [B, N, H_q, d]
    k: np.ndarray  # stored keys [B, N, H_kv, d], unit norm
    v: np.ndarray  # [B, N, H_kv, d]
    lq: np.ndarray  # log-gates [B, N, H_kv]
    lk: np.ndarray
    lb: np.ndarray
    dO: np.ndarray  # gradient of the attention output [B, N, H_q, d]

    def astuple(self):
        return self.q, self.k, self.v, self.lq, self.lk, self.lb, self.dO


def make_grad_inputs(B: int, N: int, H_q: int, H_kv: int, d: int, bf16: bool = True, seed: int = 0,
                     repeat_pairs: int = 0) -> GradInputs:
    """Seeded inputs of the attention backward.

    Queries, values and dO are N(0, 1); keys are Gaussian draws scaled to unit
    norm (RoPE keeps a key's norm); each log-gate is log sigmoid(z) of a
    pre-activation z ~ N(b_h, 32) (hidden 2048 against gate weights of variance
    1/64) with a per-head bias b_h uniform in [-4, 0], the 1B-shape prefill's
    gate statistics.  ``repeat_pairs`` copies that many keys onto later tokens
    of the same head at 1.0625 times their norm (a repeated key's similarity
    then exceeds 1).  In bf16 every q, k, v value is bf16-exact.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    q = rng.normal(0, 1, (B, N, H_q, d)).astype(np.float32)
    k = rng.normal(0, 1, (B, N, H_kv, d))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.normal(0, 1, (B, N, H_kv, d)).astype(np.float32)
    if bf16:
        q, k, v = bf16_exact(q), bf16_exact(k), bf16_exact(v)
    for _ in range(repeat_pairs):
        b, h = rng.integers(B), rng.integers(H_kv)
        t, j = sorted(rng.choice(N, 2, replace=False))
        k[b, t, h] = k[b, j, h] * np.float32(1.0625)
        if bf16:
            k[b, t, h] = bf16_exact(k[b, t, h])
    bias = rng.uniform(-4, 0, (3, H_kv))
    gates = []
    for g in range(3):
        z = rng.normal(0, math.sqrt(32.0), (B, N, H_kv)) + bias[g]
        gates.append((-np.logaddexp(0.0, -z)).astype(np.float32))
    dO = rng.normal(0, 1, (B, N, H_q, d)).astype(np.float32)
    return GradInputs(q, k, v, gates[0], gates[1], gates[2], dO)


# ---------------------------------------------------------------------------
# caches with constructed keep masks (compaction exactness)
# ---------------------------------------------------------------------------
MASK_PATTERNS = ("dead", "live", "alt", "first_only", "last_only", "first_dead", "last_dead", "random", "front_dead")


def mask_pattern(kind: str, n: int, rng: np.random.Generator) -> np.ndarray:
    """A keep mask of n entries: every entry dead or live, alternating (the
    first live), a single survivor first or last, everything but the first
    or the last entry, a seeded coin per entry, or the first half dead (so
    every survivor moves)."""
    m = np.zeros(n, bool)
    if n == 0:
        return m
    if kind == "live":
        m[:] = True
    elif kind == "alt":
        m[0::2] = True
    elif kind == "first_only":
        m[0] = True
    elif kind == "last_only":
        m[-1] = True
    elif kind == "first_dead":
        m[1:] = True
    elif kind == "last_dead":
        m[:-1] = True
    elif kind == "random":
        m = rng.random(n) < 0.5
    elif kind == "front_dead":
        m[n // 2 :] = True
    elif kind != "dead":
        raise ValueError(kind)
    return m


def make_mask_cache(lengths, kinds, d: int, bf16: bool, log_p: float, seed: int = 0, extra: int = 16,
                    B: Optional[int] = None) -> CacheInit:
    """A cache whose segment s holds lengths[s] entries with keep mask kinds[s].

    Live entries get log-biases uniform in [log_p + 1e-3, 0], dead ones
    uniform in [log_p - 2, log_p - 1e-3] (every decision is 1e-3 or more
    away from the threshold); keys, values and key gates are N(0, 1) draws
    (bf16-exact in bf16 caches), distinct per row so a misplaced row shows.
    ``B`` sequences share the segments evenly (default: one KV head each).
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    lengths = np.asarray(lengths, np.int64)
    S = lengths.size
    off, cap, slots = make_layout(lengths, extra)
    K = rng.standard_normal((slots, d), dtype=np.float32)
    V = rng.standard_normal((slots, d), dtype=np.float32)
    lk = -np.abs(rng.standard_normal(slots, dtype=np.float32))
    lam = np.zeros(slots, np.float32)
    for s in range(S):
        n = int(lengths[s])
        m = mask_pattern(kinds[s], n, rng)
        live = rng.uniform(log_p + 1e-3, 0.0, n)
        dead = rng.uniform(log_p - 2.0, log_p - 1e-3, n)
        lam[off[s] : off[s] + n] = np.where(m, live, dead).astype(np.float32)
    if bf16:
        K, V = bf16_exact(K), bf16_exact(V)
    nb = S if B is None else B
    return CacheInit(K=K, V=V, lam=lam, lk=lk, seg_off=off, seg_len=lengths.astype(np.int32), seg_cap=cap,
                     next_pos=np.zeros(nb, np.int32))
