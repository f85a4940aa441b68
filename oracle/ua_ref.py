"""fp64 reference ("oracle") for one Universal Attention (UA) layer.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the pages this follows; no equations survive on them, so every exact
form below is a reading, listed at the end of this docstring):

* paperlayer.ai summary, section 3 "Softmax multi-head self-attention":
  causal softmax attention over L tokens, n heads, head dim d; keys and values
  of past tokens are kept per layer (the KV cache).
* same page, section 3 "Data dependent forget-gates": FoX turns a per-token
  scalar gate into an additive bias on the attention matrix whose accumulated
  decay falls monotonically away from the diagonal.
* same page, section 4: the decay mechanisms are combined by a geometric mean
  into one decay rate per position pair.
* same page, section 4.1: a query-axis and a key-axis first-order statistic and
  a pairwise (key-similarity) second-order term; the key-aware rate is fixed
  per token; the similarity term is a multiplicative DeltaNet-style factor.
* same page, section 4.2: at inference a KV pair is evicted once its effective
  mask falls below p, per head; the bias only decreases.
* ai4snews page, Figure 1 caption: keys are L2-normalised, RoPE is kept, a
  low-rank sigmoid gate multiplies the attention output, and the bias matrix
  Lambda comes from the three terms in three moves: their geometric mean,
  then its logarithm, then a causal running sum.
* ai4snews page, paragraph after Figure 1: the geometric mean vetoes (one term
  saying "no decay" zeroes the combined decay); f_q alone is FoX-style; one
  scalar bias is kept per KV pair and eviction is monotone.

Specification (both this oracle and the GPU path follow it)
-----------------------------------------------------------
Parameters: W_dec [D, 3*H_kv] (column m*H_kv + h; m = 0 query gate, 1 key
gate, 2 similarity gate), b_dec [3*H_kv]; W_dn [D, r]; W_up [r, H_q*d];
b_up [H_q*d]; sm_scale (default d**-0.5); theta = rope_base; the set S of
enabled terms (subset of {q, k, sim}); tau = log p, p in [0, 1), tau = -inf
when p = 0.

O1 keys      k_hat = k / max(||k||_2, 1e-12)
O2 RoPE      rotate-half: for i < d/2, w_i = theta**(-2i/d), phi = pos*w_i,
             (x_i, x_{i+d/2}) -> (x_i cos phi - x_{i+d/2} sin phi,
                                  x_{i+d/2} cos phi + x_i sin phi).
             q~ = RoPE(q); k~ = round_cache(RoPE(k_hat)) (bf16 round to
             nearest even for a bf16 cache, identity for an fp32 cache).
O3 gates     z = x W_dec + b_dec; per KV head h: lq = logsig(z[h]),
             lk = logsig(z[H_kv + h]), lb = logsig(z[2 H_kv + h]).
O4 pair term (j < t) s = <k~_t, k~_j>, u = min(s^2, 1);
             L_q = lq_t, L_k = lk_j, L_sim = lb_t + log u;
             lambda = mean over m in S of L_m;  A_tj = log(1 - exp(lambda)).
             S empty -> A = 0; lambda = -inf -> A = 0; lambda = 0 -> A = -inf.
O5 bias      Lambda_ij = sum_{t=j+1..i} A_tj (so Lambda_ii = 0).
O6 live      live_i = {j <= i : Lambda_ij >= tau}.
O7 attention for query head a of KV group h = a // G:
             e_ij = sm_scale <q~_i^a, k~_j> + Lambda_ij over live j,
             P = softmax_j(e), o_i^a = sum_j P_ij v_j^h.
O8 gate      gamma_i = sigmoid((x_i W_dn) W_up + b_up) viewed as [H_q, d];
             y_i = gamma_i * o_i.

Decode step for one token per sequence: O1-O3 at pos = next_pos[b]; for
every cached entry that is still live (Lambda_j >= tau) add A_tj to
Lambda_j; entries whose new Lambda_j < tau die now and are not attended;
append (k~_t, v_t, Lambda = 0, lk_t) unless the segment is full (then a
sticky status bit is set and the append skipped; the token still attends to
itself); attend over the live entries plus the new one; next_pos[b] += 1.
Entries that were already dead before the step are skipped, so the result
does not depend on how often compaction runs.

Prefill of n tokens: the same per-token update with tau = -inf (dense within
the call); the cache's Lambda vector at the end is the final per-KV bias.

Compaction: per segment, stable removal of entries with Lambda < tau; the
kept-index list holds the pre-compaction in-segment indices of survivors.

Readings where the pages are silent (both paths follow them)
-------------------------------------------------------------
R1  f_sim decay amount = beta_t * min(s^2, 1) with beta_t = sigmoid(z_sim):
    the retention a DeltaNet write (I - beta k_t k_t^T) leaves along a unit
    key k_j is 1 - beta s^2, so the decay is beta s^2 (zero for orthogonal
    keys, which makes the veto meaningful).
R2  all three decay gates project the layer input x through W_dec + b_dec;
    q/k/v are given (their projections lie outside the layer kernel).
R3  lk_j is computed once when entry j is inserted and stored with it.
R4  the geometric mean is taken over decay amounts delta_m in [0, 1) with
    exponent 1/|S| over the enabled terms only (so f_q alone is FoX).
R5  "log-space" = log-retention A = log(1 - delta) <= 0.
R6  the sum runs over t = j+1..i (Lambda_ii = 0).
R7  similarity uses the stored (RoPE'd, normalised, cache-dtype) keys.
R8  gates and Lambda are per KV head; the G query heads of a group share them.
R9  RoPE angles are formed in fp64; no frequency scaling.
R10 sm_scale = d**-0.5 unless given.
R11 output gate is elementwise over [H_q, d] with rank r, b_up default 0.
R12 evict-then-attend: an entry whose updated Lambda < tau is not attended.
R13 live iff Lambda >= tau (ties keep); the new entry is always live.
R14 prefill is dense inside a call; eviction is a separate compaction.
R15 positions: prefill pos = next_pos + i; decode pos = next_pos.
R16 logsig and log1mexp are evaluated stably (Maechler 2012 for log1mexp).
R17 for parity the harness may hand this oracle the GPU-stored k~ bits
    (after checking they are within one bf16 ulp of its own rounding).
R26 "Qwen3-style normalized queries and keys" (paperlayer.ai summary,
    Appendix E, ablations) = RMS normalisation over the head dimension with
    a learned per-dimension weight shared by the heads, x / sqrt(mean(x^2) +
    eps) * w with eps = 1e-6, applied to the projected q and k before O1-O2
    (so the key is still L2-normalised afterwards).  It is an optional step
    in front of the layer; the result is rounded to the token dtype.
R31 variable-length prefill: sequence b appends its own n_b tokens (packed
    rows cu[b] .. cu[b+1]); sequences share nothing (each KV segment belongs
    to one sequence: paperlayer.ai section 4.2), so the call is R14's prefill
    of each sequence on its own, n_b = 0 leaving it untouched.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence

import numpy as np

TERM_Q = 1
TERM_K = 2
TERM_SIM = 4
TERMS_ALL = TERM_Q | TERM_K | TERM_SIM

_LN2 = math.log(2.0)


# ---------------------------------------------------------------------------
# configuration containers
# ---------------------------------------------------------------------------
@dataclass
class Dims:
    """Layer shape.  G = H_q // H_kv query heads share one KV head."""

    B: int
    H_q: int
    H_kv: int
    d: int
    D: int
    r: int = 16
    terms: int = TERMS_ALL
    rope_base: float = 10000.0
    sm_scale: float = 0.0  # 0 -> d ** -0.5
    cache_bf16: bool = True

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale != 0.0 else 1.0 / math.sqrt(self.d)


@dataclass
class Params:
    """Layer weights as fp64 arrays (values exactly as the GPU sees them)."""

    W_dec: np.ndarray  # [D, 3*H_kv]
    b_dec: np.ndarray  # [3*H_kv]
    W_dn: np.ndarray  # [D, r]
    W_up: np.ndarray  # [r, H_q*d]
    b_up: Optional[np.ndarray] = None  # [H_q*d] or None (= 0)


@dataclass
class RefCache:
    """Per-(b, h_kv) segment lists of cache entries, in insertion order."""

    K: List[np.ndarray]  # segment s = b*H_kv + h : [n_s, d]
    V: List[np.ndarray]
    lam: List[np.ndarray]  # [n_s]  log-bias Lambda_j
    lk: List[np.ndarray]  # [n_s]  key gate logsig(z_k) fixed at insertion
    next_pos: np.ndarray  # [B] int64
    cap: np.ndarray  # [B*H_kv] capacity per segment
    status: int = 0

    @staticmethod
    def empty(dims: Dims, cap: Sequence[int], next_pos: Optional[Sequence[int]] = None) -> "RefCache":
        S = dims.B * dims.H_kv
        return RefCache(
            K=[np.zeros((0, dims.d)) for _ in range(S)],
            V=[np.zeros((0, dims.d)) for _ in range(S)],
            lam=[np.zeros(0) for _ in range(S)],
            lk=[np.zeros(0) for _ in range(S)],
            next_pos=np.zeros(dims.B, np.int64) if next_pos is None else np.asarray(next_pos, np.int64).copy(),
            cap=np.asarray(cap, np.int64).copy(),
        )

    def copy(self) -> "RefCache":
        return RefCache(
            K=[a.copy() for a in self.K],
            V=[a.copy() for a in self.V],
            lam=[a.copy() for a in self.lam],
            lk=[a.copy() for a in self.lk],
            next_pos=self.next_pos.copy(),
            cap=self.cap.copy(),
            status=self.status,
        )

    def lengths(self) -> np.ndarray:
        return np.array([a.shape[0] for a in self.lam], np.int64)


# ---------------------------------------------------------------------------
# elementary functions (Figure 1 caption of the ai4snews page; section 4.1)
# ---------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and fp32's exponent range; the rounding
    is done straight from fp64 (no intermediate fp32 rounding).
    """
    x = np.asarray(x, np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    xf = x[fin]
    _, e = np.frexp(xf)  # xf = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)  # quantum exponent; -133 = bf16 subnormal step
    scaled = np.ldexp(xf, -q)  # exact (power-of-two scaling)
    rounded = np.ldexp(np.round(scaled), q)  # np.round: ties to even
    big = np.abs(rounded) > 3.3895313892515355e38  # largest finite bf16
    rounded[big] = np.copysign(np.inf, rounded[big])
    out[fin] = rounded
    return out


def l2_normalize(k: np.ndarray) -> np.ndarray:
    """O1: k / max(||k||_2, 1e-12) along the last axis (Figure 1 caption)."""
    k = np.asarray(k, np.float64)
    n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    return k / np.maximum(n, 1e-12)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """O2: rotate-half RoPE of the last axis at position ``pos`` (fp64).

    ``x`` is [..., d]; ``pos`` broadcasts against x's leading axes.
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    w = base ** (-2.0 * i / d)
    phi = np.asarray(pos, np.float64)[..., None] * w
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def log_sigmoid(z: np.ndarray) -> np.ndarray:
    """O3: log(sigmoid(z)) = -softplus(-z), evaluated without overflow."""
    z = np.asarray(z, np.float64)
    return -(np.maximum(-z, 0.0) + np.log1p(np.exp(-np.abs(z))))


def log1mexp(lam: np.ndarray) -> np.ndarray:
    """O4: log(1 - exp(lam)) for lam <= 0 (Maechler 2012, switch at -ln 2)."""
    lam = np.asarray(lam, np.float64)
    out = np.empty_like(lam)
    near = lam > -_LN2
    with np.errstate(divide="ignore"):
        out[near] = np.log(-np.expm1(lam[near]))
    out[~near] = np.log1p(-np.exp(lam[~near]))
    return out


def qk_rmsnorm(x: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """R26: x / sqrt(mean(x^2) + eps) * w along the last (head) axis."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, np.float64)


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, np.float64)
    return np.where(z >= 0, 1.0 / (1.0 + np.exp(-np.abs(z))), np.exp(-np.abs(z)) / (1.0 + np.exp(-np.abs(z))))


# ---------------------------------------------------------------------------
# per-token quantities
# ---------------------------------------------------------------------------
def gates(dims: Dims, params: Params, x: np.ndarray):
    """O3: (lq, lk, lb) per KV head for token input(s) x [..., D]."""
    z = np.asarray(x, np.float64) @ params.W_dec + params.b_dec
    H = dims.H_kv
    return log_sigmoid(z[..., 0:H]), log_sigmoid(z[..., H : 2 * H]), log_sigmoid(z[..., 2 * H : 3 * H])


def output_gate(dims: Dims, params: Params, x: np.ndarray) -> np.ndarray:
    """O8: gamma = sigmoid((x W_dn) W_up + b_up), shaped [..., H_q, d]."""
    u = np.asarray(x, np.float64) @ params.W_dn
    g = u @ params.W_up
    if params.b_up is not None:
        g = g + params.b_up
    return sigmoid(g).reshape(g.shape[:-1] + (dims.H_q, dims.d))


def round_cache(dims: Dims, k: np.ndarray) -> np.ndarray:
    return bf16_round(k) if dims.cache_bf16 else np.asarray(k, np.float64)


def preprocess_token(dims: Dims, params: Params, q, k, x, pos):
    """O1-O3 and O8's gate for one token of one sequence.

    q [H_q, d], k [H_kv, d], x [D] -> (q~ [H_q, d], k~ [H_kv, d],
    lq, lk, lb [H_kv], gamma [H_q, d]).
    """
    qt = rope(q, np.full(dims.H_q, pos), dims.rope_base)
    kt = round_cache(dims, rope(l2_normalize(k), np.full(dims.H_kv, pos), dims.rope_base))
    lq, lk, lb = gates(dims, params, x)
    gamma = output_gate(dims, params, x)
    return qt, kt, lq, lk, lb, gamma


def pair_term(terms: int, kt_t: np.ndarray, K: np.ndarray, lq_t: float, lk: np.ndarray, lb_t: float) -> np.ndarray:
    """O4: A_tj for a new key k~_t against stored keys K [n, d] (R1, R4, R5).

    ``lk`` [n] are the stored key gates of the entries.
    """
    n = K.shape[0]
    if terms == 0 or n == 0:
        return np.zeros(n)
    acc = np.zeros(n)
    cnt = 0
    if terms & TERM_Q:
        acc = acc + lq_t
        cnt += 1
    if terms & TERM_K:
        acc = acc + lk
        cnt += 1
    if terms & TERM_SIM:
        s = K @ kt_t
        u = np.minimum(s * s, 1.0)
        with np.errstate(divide="ignore"):
            acc = acc + (lb_t + np.log(u))
        cnt += 1
    lam = acc / cnt
    return log1mexp(lam)


def attend(qt_group: np.ndarray, K: np.ndarray, V: np.ndarray, lam: np.ndarray, scale: float) -> np.ndarray:
    """O7 for one KV group: q~ [G, d] against entries K, V [n, d], bias lam [n]."""
    e = scale * (qt_group @ K.T) + lam[None, :]
    m = np.max(e, axis=1, keepdims=True)
    p = np.exp(e - m)
    p = p / np.sum(p, axis=1, keepdims=True)
    return p @ V


# ---------------------------------------------------------------------------
# decode step, prefill, compaction (section 4.2 of the paperlayer.ai page)
# ---------------------------------------------------------------------------
def _tau(log_p: float) -> float:
    return -math.inf if log_p == -math.inf else float(log_p)


def decode_step(
    dims: Dims,
    params: Params,
    cache: RefCache,
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    x: np.ndarray,
    log_p: float,
    decide: Optional[Callable[[int, np.ndarray, np.ndarray], np.ndarray]] = None,
    k_override: Optional[np.ndarray] = None,
):
    """One UA decode step for every sequence; updates ``cache`` in place.

    q [B, H_q, d], k/v [B, H_kv, d], x [B, D]; log_p = log threshold (or -inf).
    ``decide(s, lam_new, idx)`` may replace the live decision for the updated
    entries of segment s (the parity harness adopts the GPU's choice for
    entries within 1e-4 of tau); ``k_override`` [B, H_kv, d] replaces the
    stored new keys (R17).  Returns y [B, H_q, d] and a per-segment info list.
    """
    tau = _tau(log_p)
    G = dims.G
    y = np.zeros((dims.B, dims.H_q, dims.d))
    info = []
    for b in range(dims.B):
        pos = int(cache.next_pos[b])
        qt, kt, lq, lk, lb, gamma = preprocess_token(dims, params, q[b], k[b], x[b], pos)
        if k_override is not None:
            kt = np.asarray(k_override[b], np.float64)
        for h in range(dims.H_kv):
            s = b * dims.H_kv + h
            K, V, lam, lks = cache.K[s], cache.V[s], cache.lam[s], cache.lk[s]
            alive_before = lam >= tau
            idx = np.flatnonzero(alive_before)
            A = pair_term(dims.terms, kt[h], K[idx], lq[h], lks[idx], lb[h])
            lam = lam.copy()
            lam[idx] = lam[idx] + A
            live_new = lam[idx] >= tau
            if decide is not None:
                live_new = np.asarray(decide(s, lam[idx], idx), bool)
            att = idx[live_new]
            # the new token attends to itself whether or not it is stored
            Katt = np.vstack([K[att], kt[h][None, :]])
            Vatt = np.vstack([V[att], np.asarray(v[b, h], np.float64)[None, :]])
            latt = np.concatenate([lam[att], [0.0]])
            o = attend(qt[h * G : (h + 1) * G], Katt, Vatt, latt, dims.scale)
            y[b, h * G : (h + 1) * G] = gamma[h * G : (h + 1) * G] * o
            # dead entries keep the Lambda they fell to; they are never revived
            cache.lam[s] = lam
            full = K.shape[0] >= cache.cap[s]
            if full:
                cache.status |= 1
            else:
                cache.K[s] = np.vstack([K, kt[h][None, :]])
                cache.V[s] = np.vstack([V, np.asarray(v[b, h], np.float64)[None, :]])
                cache.lam[s] = np.concatenate([lam, [0.0]])
                cache.lk[s] = np.concatenate([lks, [lk[h]]])
            info.append({"seg": s, "updated_idx": idx, "lam_updated": lam[idx], "live": live_new, "A": A})
        cache.next_pos[b] = pos + 1
    return y, info


def prefill(
    dims: Dims,
    params: Params,
    cache: RefCache,
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    x: np.ndarray,
    k_override: Optional[np.ndarray] = None,
) -> np.ndarray:
    """Dense prefill of n tokens per sequence by the row recurrence (R14).

    q [B, n, H_q, d], k/v [B, n, H_kv, d], x [B, n, D] -> y [B, n, H_q, d].
    Token i updates every cached Lambda_j by A_ij, is appended, then attends
    to the whole cache (tau = -inf): exactly O5-O8 with Lambda_ii = 0.
    ``k_override`` [B, n, H_kv, d] supplies stored key bits (R17).
    """
    n = q.shape[1]
    y = np.zeros((dims.B, n, dims.H_q, dims.d))
    for i in range(n):
        ko = None if k_override is None else k_override[:, i]
        yi, _ = decode_step(dims, params, cache, q[:, i], k[:, i], v[:, i], x[:, i], -math.inf, k_override=ko)
        y[:, i] = yi
    return y


def prefill_varlen(
    dims: Dims,
    params: Params,
    cache: RefCache,
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    x: np.ndarray,
    cu: Sequence[int],
    k_override: Optional[np.ndarray] = None,
) -> np.ndarray:
    """Variable-length prefill (R31): packed rows cu[b] .. cu[b+1] of q [T, H_q, d],
    k/v [T, H_kv, d], x [T, D] are sequence b's tokens; returns y [T, H_q, d]."""
    T = q.shape[0]
    y = np.zeros((T, dims.H_q, dims.d))
    H = dims.H_kv
    for b in range(dims.B):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 <= r0:
            continue
        segs = slice(b * H, (b + 1) * H)
        one = Dims(B=1, H_q=dims.H_q, H_kv=H, d=dims.d, D=dims.D, r=dims.r, terms=dims.terms,
                   rope_base=dims.rope_base, sm_scale=dims.sm_scale, cache_bf16=dims.cache_bf16)
        sub = RefCache(K=cache.K[segs], V=cache.V[segs], lam=cache.lam[segs], lk=cache.lk[segs],
                       next_pos=cache.next_pos[b : b + 1].copy(), cap=cache.cap[segs].copy())
        ko = None if k_override is None else k_override[None, r0:r1]
        y[r0:r1] = prefill(one, params, sub, q[None, r0:r1], k[None, r0:r1], v[None, r0:r1], x[None, r0:r1],
                           k_override=ko)[0]
        cache.K[segs], cache.V[segs], cache.lam[segs], cache.lk[segs] = sub.K, sub.V, sub.lam, sub.lk
        cache.next_pos[b] = sub.next_pos[0]
        cache.status |= sub.status
    return y


def compact(cache: RefCache, log_p: float) -> List[np.ndarray]:
    """Stable in-place removal of entries with Lambda < tau, per segment.

    Returns the kept (pre-compaction, in-segment) indices of every segment.
    """
    tau = _tau(log_p)
    kept_all = []
    for s in range(len(cache.lam)):
        kept = np.flatnonzero(cache.lam[s] >= tau)
        cache.K[s] = cache.K[s][kept]
        cache.V[s] = cache.V[s][kept]
        cache.lam[s] = cache.lam[s][kept]
        cache.lk[s] = cache.lk[s][kept]
        kept_all.append(kept)
    return kept_all


# ---------------------------------------------------------------------------
# dense forms of O5 / O7 for a single (b, h_kv) sequence (used by the pins
# and for sampled rows at large sizes)
# ---------------------------------------------------------------------------
def dense_logbias(terms: int, Kt: np.ndarray, lq: np.ndarray, lk: np.ndarray, lb: np.ndarray, rows=None) -> np.ndarray:
    """O5 as column sums: Lambda [len(rows), N] for stored keys Kt [N, d].

    Lambda_ij = sum_{t=j+1..i} A_tj; entries j > i are -inf (causal mask).
    Built row by row (A_t. for t = 1..max row), one library matmul per row.
    """
    N = Kt.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    need = int(rows.max()) if rows.size else -1
    col = np.zeros(N)
    out = np.full((rows.size, N), -np.inf)
    want = {}
    for i, r in enumerate(rows):
        want.setdefault(int(r), []).append(i)  # a row may be asked for more than once
    for t in range(0, need + 1):
        if t > 0:
            col[:t] += pair_term(terms, Kt[t], Kt[:t], lq[t], lk[:t], lb[t])
        for i in want.get(t, ()):
            out[i, : t + 1] = col[: t + 1]
    return out


def dense_attention(qt: np.ndarray, Kt: np.ndarray, V: np.ndarray, lam_rows: np.ndarray, rows: np.ndarray, scale: float) -> np.ndarray:
    """O7 for sampled rows of one KV group: qt [N, G, d] -> o [len(rows), G, d]."""
    out = np.zeros((len(rows), qt.shape[1], qt.shape[2]))
    for ri, i in enumerate(rows):
        i = int(i)
        out[ri] = attend(qt[i], Kt[: i + 1], V[: i + 1], lam_rows[ri, : i + 1], scale)
    return out
