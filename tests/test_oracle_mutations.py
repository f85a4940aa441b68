"""Planted mistakes in the oracle (CPU only) must each fail at least one pin.

Every mutation below is a plausible slip in writing the method down: a dropped
or mis-weighted term, a wrong sign, a wrong frequency, a missing clamp, a
swapped gate column.  The pins in test_oracle_pins.py are run against the
mutated oracle and at least one of them has to fail.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.ua_ref as R
from tests import test_oracle_pins as P

_orig_pair_term = R.pair_term
_orig_rope = R.rope
_orig_gates = R.gates


def _pair_sum(terms, kt_t, K, lq_t, lk, lb_t):
    """geometric mean replaced by a product (sum of logs)"""
    n = K.shape[0]
    if terms == 0 or n == 0:
        return np.zeros(n)
    acc = np.zeros(n)
    if terms & R.TERM_Q:
        acc = acc + lq_t
    if terms & R.TERM_K:
        acc = acc + lk
    if terms & R.TERM_SIM:
        s = K @ kt_t
        with np.errstate(divide="ignore"):
            acc = acc + lb_t + np.log(np.minimum(s * s, 1.0))
    return R.log1mexp(acc)


def _pair_mean_over_three(terms, kt_t, K, lq_t, lk, lb_t):
    """exponent 1/3 even when fewer terms are enabled"""
    n = K.shape[0]
    if terms == 0 or n == 0:
        return np.zeros(n)
    acc = np.zeros(n)
    if terms & R.TERM_Q:
        acc = acc + lq_t
    if terms & R.TERM_K:
        acc = acc + lk
    if terms & R.TERM_SIM:
        s = K @ kt_t
        with np.errstate(divide="ignore"):
            acc = acc + lb_t + np.log(np.minimum(s * s, 1.0))
    return R.log1mexp(acc / 3.0)


def _pair_abs_s(terms, kt_t, K, lq_t, lk, lb_t):
    """|s| instead of s^2 in the similarity decay"""
    n = K.shape[0]
    if terms == 0 or n == 0:
        return np.zeros(n)
    acc, cnt = np.zeros(n), 0
    if terms & R.TERM_Q:
        acc, cnt = acc + lq_t, cnt + 1
    if terms & R.TERM_K:
        acc, cnt = acc + lk, cnt + 1
    if terms & R.TERM_SIM:
        s = K @ kt_t
        with np.errstate(divide="ignore"):
            acc, cnt = acc + lb_t + np.log(np.minimum(np.abs(s), 1.0)), cnt + 1
    return R.log1mexp(acc / cnt)


def _pair_no_clamp(terms, kt_t, K, lq_t, lk, lb_t):
    """s^2 not clamped at 1"""
    n = K.shape[0]
    if terms == 0 or n == 0:
        return np.zeros(n)
    acc, cnt = np.zeros(n), 0
    if terms & R.TERM_Q:
        acc, cnt = acc + lq_t, cnt + 1
    if terms & R.TERM_K:
        acc, cnt = acc + lk, cnt + 1
    if terms & R.TERM_SIM:
        s = K @ kt_t
        with np.errstate(divide="ignore"):
            acc, cnt = acc + lb_t + np.log(s * s), cnt + 1
    lam = np.minimum(acc / cnt, 0.0)
    return R.log1mexp(lam)


def _pair_retention_mean(terms, kt_t, K, lq_t, lk, lb_t):
    """geometric mean of retentions instead of decay amounts (no veto)"""
    n = K.shape[0]
    if terms == 0 or n == 0:
        return np.zeros(n)
    acc, cnt = np.zeros(n), 0
    if terms & R.TERM_Q:
        acc, cnt = acc + R.log1mexp(np.full(n, lq_t)), cnt + 1
    if terms & R.TERM_K:
        acc, cnt = acc + R.log1mexp(lk), cnt + 1
    if terms & R.TERM_SIM:
        s = K @ kt_t
        with np.errstate(divide="ignore"):
            acc, cnt = acc + R.log1mexp(np.minimum(lb_t + np.log(np.minimum(s * s, 1.0)), 0.0)), cnt + 1
    return acc / cnt


def _log1mexp_wrong(lam):
    """log(1 + e^lam) instead of log(1 - e^lam)"""
    return -np.log1p(np.exp(np.asarray(lam, float)))


def _rope_wrong_freq(x, pos, base):
    """frequencies base^(-i/d) instead of base^(-2i/d)"""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    w = base ** (-np.arange(half) / d)
    phi = np.asarray(pos, np.float64)[..., None] * w
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _rope_wrong_dir(x, pos, base):
    """rotation by -phi"""
    return _orig_rope(x, -np.asarray(pos, np.float64), base)


def _rope_interleaved(x, pos, base):
    """pairs (2i, 2i+1) instead of (i, i+d/2)"""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return _orig_rope(x[..., perm], pos, base)[..., inv]


def _gates_swapped(dims, params, x):
    """query and key gate columns swapped"""
    lq, lk, lb = _orig_gates(dims, params, x)
    return lk, lq, lb


def _output_gate_no_sigmoid(dims, params, x):
    u = np.asarray(x, np.float64) @ params.W_dn
    g = u @ params.W_up
    if params.b_up is not None:
        g = g + params.b_up
    return np.tanh(g).reshape(g.shape[:-1] + (dims.H_q, dims.d)) * 0.5 + 0.5


def _log_sigmoid_wrong(z):
    """log sigmoid(-z) instead of log sigmoid(z)"""
    z = np.asarray(z, np.float64)
    return -(np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z))))


def _no_normalize(k):
    return np.asarray(k, np.float64)


def _attend_no_scale(qt_group, K, V, lam, scale):
    e = qt_group @ K.T + lam[None, :]
    m = np.max(e, axis=1, keepdims=True)
    p = np.exp(e - m)
    return (p / p.sum(axis=1, keepdims=True)) @ V


MUTATIONS = {
    "pair: sum of logs": ("pair_term", _pair_sum),
    "pair: exponent 1/3 always": ("pair_term", _pair_mean_over_three),
    "pair: |s| not s^2": ("pair_term", _pair_abs_s),
    "pair: no clamp": ("pair_term", _pair_no_clamp),
    "pair: mean of retentions": ("pair_term", _pair_retention_mean),
    "log1mexp sign": ("log1mexp", _log1mexp_wrong),
    "rope frequency": ("rope", _rope_wrong_freq),
    "rope direction": ("rope", _rope_wrong_dir),
    "rope interleaved": ("rope", _rope_interleaved),
    "gates swapped": ("gates", _gates_swapped),
    "output gate": ("output_gate", _output_gate_no_sigmoid),
    "log sigmoid sign": ("log_sigmoid", _log_sigmoid_wrong),
    "no key normalisation": ("l2_normalize", _no_normalize),
    "no softmax scale": ("attend", _attend_no_scale),
}

PINS = [
    "test_pair_term_worked_examples",
    "test_rope_worked_examples",
    "test_P9_log1mexp_logsigmoid_mpmath",
    "test_P0_single_token_output_gate",
    "test_P2_query_term_is_fox",
    "test_P3_key_term_fixed_rate",
    "test_P4_similarity_term_equal_keys",
    "test_P5_key_veto_keeps_column_at_zero",
    "test_P5_orthogonal_key_not_decayed",
    "test_P7_decode_equals_dense_threshold_attention",
    "test_P8_brute_force_mpmath",
]


def _run_pin(name, golden_dir):
    fn = getattr(P, name)
    try:
        if name in ("test_pair_term_worked_examples", "test_rope_worked_examples"):
            fn(golden_dir)
        else:
            fn()
    except (AssertionError, ValueError, FloatingPointError):
        return False
    return True


@pytest.mark.parametrize("mut", sorted(MUTATIONS))
def test_mutation_is_caught(mut, monkeypatch, golden_dir):
    attr, fn = MUTATIONS[mut]
    monkeypatch.setattr(R, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    with np.errstate(all="ignore"):
        failed = [p for p in PINS if not _run_pin(p, golden_dir)]
    assert failed, f"no pin caught mutation {mut!r}"


def test_unmutated_passes_all(golden_dir):
    assert all(_run_pin(p, golden_dir) for p in PINS)
