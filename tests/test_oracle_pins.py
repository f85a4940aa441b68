"""Pins that tie the fp64 oracle to what the pages and mathematics fix.

Each test states the passage it follows.  None of them re-types an oracle
formula: they use hand-worked values (tests/golden), closed forms of special
cases, a library routine (torch SDPA, torch bf16 conversion, mpmath),
invariants, or an explicit brute force on tiny inputs.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as U

RNG = np.random.default_rng


def _dims(B=1, H_q=2, H_kv=1, d=8, D=6, r=3, terms=U.TERMS_ALL, bf16=False, base=10000.0):
    return U.Dims(B=B, H_q=H_q, H_kv=H_kv, d=d, D=D, r=r, terms=terms, rope_base=base, cache_bf16=bf16)


def _params(dims, rng, gate_scale=1.0, gamma_one=True):
    W_dec = rng.normal(0, gate_scale, (dims.D, 3 * dims.H_kv))
    b_dec = rng.normal(0, 1, 3 * dims.H_kv)
    W_dn = rng.normal(0, 1, (dims.D, dims.r))
    if gamma_one:  # sigmoid(1e3) == 1.0 exactly in fp64, so y = o
        W_up = np.zeros((dims.r, dims.H_q * dims.d))
        b_up = np.full(dims.H_q * dims.d, 1e3)
    else:
        W_up = rng.normal(0, 0.5, (dims.r, dims.H_q * dims.d))
        b_up = rng.normal(0, 0.5, dims.H_q * dims.d)
    return U.Params(W_dec=W_dec, b_dec=b_dec, W_dn=W_dn, W_up=W_up, b_up=b_up)


def _tokens(dims, n, rng):
    q = rng.normal(0, 1, (dims.B, n, dims.H_q, dims.d))
    k = rng.normal(0, 1, (dims.B, n, dims.H_kv, dims.d))
    v = rng.normal(0, 1, (dims.B, n, dims.H_kv, dims.d))
    x = rng.normal(0, 1, (dims.B, n, dims.D))
    return q, k, v, x


def _fresh(dims, cap=10_000):
    return U.RefCache.empty(dims, [cap] * (dims.B * dims.H_kv))


def _sdpa_masked(qt, kt, v, G, bias):
    """torch SDPA in fp64 on the CPU; qt [N,H_q,d], kt/v [N,H_kv,d], bias [N,N] (-inf = masked)."""
    Q = torch.tensor(qt).permute(1, 0, 2)[None]
    K = torch.tensor(kt).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    V = torch.tensor(v).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    M = torch.tensor(bias)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=M)[0].permute(1, 0, 2).numpy()


def _preprocessed(dims, params, q, k, x, pos0=0):
    """q~ and stored k~ of every token of sequence 0 via the oracle's O1/O2."""
    n = q.shape[1]
    qt = np.stack([U.rope(q[0, i], np.full(dims.H_q, pos0 + i), dims.rope_base) for i in range(n)])
    kt = np.stack(
        [U.round_cache(dims, U.rope(U.l2_normalize(k[0, i]), np.full(dims.H_kv, pos0 + i), dims.rope_base)) for i in range(n)]
    )
    return qt, kt


def _logsig_neg(z):
    """log(1 - sigmoid(z)) = -log(1 + e^z), the FoX log-forget value (moderate z only)."""
    return -np.log1p(np.exp(z))


# ---------------------------------------------------------------------------
# golden worked examples
# ---------------------------------------------------------------------------
def _val(v):
    if isinstance(v, (int, float)):
        return float(v)
    table = {"-ln3": -math.log(3), "ln3": math.log(3), "-ln8": -math.log(8), "ln(3/4)": math.log(0.75),
             "ln(1/4)": math.log(0.25), "ln(2/3)": math.log(2 / 3), "ln(1/2)": math.log(0.5), "0": 0.0}
    return table[v]


def test_pair_term_worked_examples(golden_dir):
    """Geometric mean of decay amounts, log-space, veto (section 4, 4.1; Fig. 1 caption)."""
    g = json.load(open(os.path.join(golden_dir, "pair_term_worked.json")))
    for c in g["cases"]:
        lq = U.log_sigmoid(np.array(_val(c["z_q"])))
        lk = U.log_sigmoid(np.array([_val(c["z_k"])]))
        lb = U.log_sigmoid(np.array(_val(c["z_sim"])))
        d = 4
        kt_t = np.zeros(d)
        kt_t[0] = 1.0
        kj = np.zeros((1, d))
        s = float(c["s"])
        # a stored key with <k_t, k_j> = s (norm irrelevant to the term)
        kj[0, 0] = s
        kj[0, 1] = math.sqrt(max(0.0, 1 - s * s))
        A = U.pair_term(c["terms"], kt_t, kj, float(lq), lk, float(lb))
        assert abs(A[0] - _val(c["A"])) <= 1e-14, c["name"]


def test_compaction_worked_example(golden_dir):
    """Stable eviction below log p with ties kept (section 4.2)."""
    g = json.load(open(os.path.join(golden_dir, "compact_worked.json")))
    lam = np.array([float(v) for v in g["lam"]])
    n = lam.size
    d = 3
    cache = U.RefCache(K=[np.arange(n * d, dtype=float).reshape(n, d)], V=[-np.arange(n * d, dtype=float).reshape(n, d)],
                       lam=[lam.copy()], lk=[np.arange(n, dtype=float)], next_pos=np.zeros(1, np.int64), cap=np.array([64]))
    kept = U.compact(cache, math.log(g["p"]))
    assert kept[0].tolist() == g["kept"]
    assert cache.K[0][:, 0].tolist() == [3.0 * i for i in g["kept"]]
    assert cache.lk[0].tolist() == [float(i) for i in g["kept"]]
    assert cache.lam[0].tolist() == [lam[i] for i in g["kept"]]


def test_rope_worked_examples(golden_dir):
    """Rotate-half RoPE with frequencies base^(-2i/d) (Fig. 1 caption: RoPE kept)."""
    g = json.load(open(os.path.join(golden_dir, "rope_worked.json")))
    d, base = g["d"], g["base"]
    for c in g["cases"]:
        e = np.zeros(d)
        e[c["unit"]] = 1.0
        out = U.rope(e, c["pos"], base)
        expect = np.zeros(d)
        for k, expr in c["expect"].items():
            expect[int(k)] = eval(expr.replace("^", "**"), {"cos": math.cos, "sin": math.sin})
        np.testing.assert_allclose(out, expect, atol=1e-15)


# ---------------------------------------------------------------------------
# P9: elementary functions against mpmath
# ---------------------------------------------------------------------------
def test_P9_log1mexp_logsigmoid_mpmath():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    lams = -np.concatenate([np.logspace(-300, math.log10(700), 400), [1e-300, 1e-17, 1e-8, 0.5, math.log(2), 0.7, 1.0, 30.0]])
    got = U.log1mexp(lams)
    for lam, g in zip(lams, got):
        with mp.workdps(700):  # enough digits that 1 - e^lam is exact for every lam here
            ref = mp.log(1 - mp.exp(mp.mpf(lam)))
        assert abs(g - float(ref)) <= 2e-15 * abs(float(ref)) + 1e-300, lam
    zs = np.concatenate([np.linspace(-700, 700, 301), [-1e4, 1e4, 0.0, 1e-12, -1e-12, 36.0, 38.0]])
    got = U.log_sigmoid(zs)
    for z, g in zip(zs, got):
        with mp.workdps(700):
            ref = -mp.log(1 + mp.exp(-mp.mpf(z)))
        assert abs(g - float(ref)) <= 2e-15 * abs(float(ref)) + 1e-320, z
    assert U.log1mexp(np.array([0.0]))[0] == -math.inf
    assert U.log1mexp(np.array([-math.inf]))[0] == 0.0


def test_bf16_round_matches_torch():
    """The oracle's own bf16 rounding equals torch's fp32->bf16 (RNE) on fp32 values."""
    rng = RNG(1)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-30, 2000), rng.normal(0, 1e30, 2000),
                        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2**-130, 3.3e38, 3.4e38])])
    x32 = x.astype(np.float32).astype(np.float64)
    ref = torch.tensor(x32, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    got = U.bf16_round(x32)
    assert np.array_equal(got, ref)
    assert U.bf16_round(np.array([1 + 2**-8]))[0] == 1.0
    assert U.bf16_round(np.array([1 + 3 * 2**-8]))[0] == 1 + 2**-6


# ---------------------------------------------------------------------------
# P0 / P1: closed forms and library attention
# ---------------------------------------------------------------------------
def test_P0_single_token_output_gate():
    """N = 1: y = gamma * v (O7 over one entry, O8), with hand-set gamma."""
    dims = _dims(B=2, H_q=4, H_kv=2, d=4, D=3, r=2)
    rng = RNG(0)
    p = _params(dims, rng)
    # gamma[a, i] = sigmoid(log(m)) = m / (m + 1) with m = a*d + i + 1
    m = np.arange(dims.H_q * dims.d, dtype=float) + 1
    p.W_up = np.zeros_like(p.W_up)
    p.b_up = np.log(m)
    q, k, v, x = _tokens(dims, 1, rng)
    y, _ = U.decode_step(dims, p, _fresh(dims), q[:, 0], k[:, 0], v[:, 0], x[:, 0], math.log(0.15))
    gam = (m / (m + 1)).reshape(dims.H_q, dims.d)
    for b in range(dims.B):
        for a in range(dims.H_q):
            np.testing.assert_allclose(y[b, a], gam[a] * v[b, 0, a // dims.G], rtol=1e-14)
    # low-rank path: x = e_0, W_dn[0, 0] = 1, W_up[0, :] = ln 3 -> gamma = 3/4
    p2 = _params(dims, rng)
    p2.W_dn = np.zeros_like(p2.W_dn)
    p2.W_dn[0, 0] = 1.0
    p2.W_up = np.zeros_like(p2.W_up)
    p2.W_up[0, :] = math.log(3)
    p2.b_up = None
    x2 = np.zeros_like(x[:, 0])
    x2[:, 0] = 1.0
    y2, _ = U.decode_step(dims, p2, _fresh(dims), q[:, 0], k[:, 0], v[:, 0], x2, math.log(0.15))
    for b in range(dims.B):
        for a in range(dims.H_q):
            np.testing.assert_allclose(y2[b, a], 0.75 * v[b, 0, a // dims.G], rtol=1e-14)


@pytest.mark.parametrize("G,H_kv", [(1, 1), (2, 2), (3, 1)])
def test_P1_no_terms_is_causal_softmax(G, H_kv):
    """All decays off: Lambda = 0 and the layer is causal softmax attention (section 3)."""
    dims = _dims(H_q=G * H_kv, H_kv=H_kv, d=8, terms=0)
    rng = RNG(10 + G)
    p = _params(dims, rng)
    n = 17
    q, k, v, x = _tokens(dims, n, rng)
    cache = _fresh(dims)
    y = U.prefill(dims, p, cache, q, k, v, x)
    for s in range(H_kv):
        assert np.all(cache.lam[s] == 0.0)
    qt, kt = _preprocessed(dims, p, q, k, x)
    Q = torch.tensor(qt).permute(1, 0, 2)[None]
    K = torch.tensor(kt).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    V = torch.tensor(v[0]).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(y[0], ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# P2 / P3 / P4: single-term closed forms
# ---------------------------------------------------------------------------
def _single_term_case(terms, seed, equal_keys=False):
    dims = _dims(H_q=2, H_kv=1, d=8, terms=terms)
    rng = RNG(seed)
    p = _params(dims, rng)
    n = 21
    q, k, v, x = _tokens(dims, n, rng)
    if equal_keys:  # pre-RoPE keys R_{-t} e_0, so every stored key is e_0
        e0 = np.zeros(dims.d)
        e0[0] = 1.0
        for i in range(n):
            k[0, i, 0] = U.rope(e0, -i, dims.rope_base) * (1.0 + i)
    cache = _fresh(dims)
    y = U.prefill(dims, p, cache, q, k, v, x)
    z = x[0] @ p.W_dec + p.b_dec  # [n, 3]
    return dims, p, q, k, v, x, cache, y, z


def _check_bias_and_output(dims, p, q, k, v, x, cache, y, Lam):
    n = Lam.shape[0]
    np.testing.assert_allclose(cache.lam[0], Lam[n - 1], rtol=1e-12, atol=1e-12)
    qt, kt = _preprocessed(dims, p, q, k, x)
    bias = np.where(np.tril(np.ones((n, n))) > 0, Lam, -np.inf)
    ref = _sdpa_masked(qt * 1.0, kt, v[0], dims.G, bias)
    np.testing.assert_allclose(y[0], ref, rtol=1e-11, atol=1e-12)


def test_P2_query_term_is_fox():
    """f_q alone = FoX: Lambda_ij = c_i - c_j, c = cumsum log(1 - sigmoid(z_q)) (ai4snews: 'FoX-style')."""
    dims, p, q, k, v, x, cache, y, z = _single_term_case(U.TERM_Q, 3)
    c = np.cumsum(_logsig_neg(z[:, 0]))
    Lam = c[:, None] - c[None, :]
    _check_bias_and_output(dims, p, q, k, v, x, cache, y, Lam)


def test_P3_key_term_fixed_rate():
    """f_k alone: each key decays at its own fixed rate, Lambda_ij = (i-j) log(1 - sigmoid(z_k,j)) (section 4.1)."""
    dims, p, q, k, v, x, cache, y, z = _single_term_case(U.TERM_K, 4)
    n = z.shape[0]
    i = np.arange(n)
    Lam = (i[:, None] - i[None, :]) * _logsig_neg(z[:, 1])[None, :]
    _check_bias_and_output(dims, p, q, k, v, x, cache, y, Lam)


def test_P4_similarity_term_equal_keys():
    """f_sim alone with identical stored keys (s = 1): Lambda_ij = sum_{t=j+1..i} log(1 - beta_t)."""
    dims, p, q, k, v, x, cache, y, z = _single_term_case(U.TERM_SIM, 5, equal_keys=True)
    c = np.cumsum(_logsig_neg(z[:, 2]))
    Lam = c[:, None] - c[None, :]
    _check_bias_and_output(dims, p, q, k, v, x, cache, y, Lam)


# ---------------------------------------------------------------------------
# P5: veto (ai4snews page, paragraph after Figure 1)
# ---------------------------------------------------------------------------
def _veto_setup(seed):
    dims = _dims(H_q=2, H_kv=1, d=8, D=6)
    rng = RNG(seed)
    p = _params(dims, rng)
    # coordinate 5 of x drives only the gate selected below
    p.W_dec[5, :] = 0.0
    p.W_dn[5, :] = 0.0
    n = 15
    q, k, v, x = _tokens(dims, n, rng)
    x[..., 5] = 0.0
    return dims, p, q, k, v, x


def test_P5_key_veto_keeps_column_at_zero():
    dims, p, q, k, v, x = _veto_setup(6)
    p.W_dec[5, 1] = 1.0  # key gate of head 0
    j = 4
    x[0, j, 5] = -1e4
    cache = _fresh(dims)
    U.prefill(dims, p, cache, q, k, v, x)
    assert cache.lam[0][j] == 0.0
    others = np.delete(cache.lam[0][:-1], j)
    assert np.all(others < 0.0)


def test_P5_query_veto_row_adds_nothing():
    dims, p, q, k, v, x = _veto_setup(7)
    p.W_dec[5, 0] = 1.0  # query gate of head 0
    t = 9
    x[0, t, 5] = -1e4
    cache = _fresh(dims)
    before = None
    for i in range(q.shape[1]):
        if i == t:
            before = cache.lam[0].copy()
        U.decode_step(dims, p, cache, q[:, i], k[:, i], v[:, i], x[:, i], -math.inf)
        if i == t:
            assert np.array_equal(cache.lam[0][:-1], before)
        elif i > 0:
            assert np.all(cache.lam[0][: i - 1] <= 0.0)


def test_P5_orthogonal_key_not_decayed():
    """A key orthogonal (after RoPE) to every later key is vetoed by f_sim."""
    dims = _dims(H_q=2, H_kv=1, d=8)
    rng = RNG(8)
    p = _params(dims, rng)
    n = 12
    q, k, v, x = _tokens(dims, n, rng)
    j = 3
    for i in range(n):
        e = np.zeros(dims.d)
        e[1 if i == j else 0] = 1.0
        k[0, i, 0] = U.rope(e, -i, dims.rope_base)
    cache = _fresh(dims)
    U.prefill(dims, p, cache, q, k, v, x)
    assert abs(cache.lam[0][j]) < 1e-9
    assert np.all(np.delete(cache.lam[0][:-1], j) < -1e-3)


# ---------------------------------------------------------------------------
# P6: monotone bias, evicted never return (section 4.2)
# ---------------------------------------------------------------------------
def test_P6_monotone_and_no_return():
    dims = _dims(B=2, H_q=4, H_kv=2, d=8, D=5)
    rng = RNG(9)
    p = _params(dims, rng, gate_scale=2.0, gamma_one=False)
    n = 40
    q, k, v, x = _tokens(dims, n, rng)
    tau = math.log(0.15)
    cache = _fresh(dims)
    prev = [np.zeros(0) for _ in range(dims.B * dims.H_kv)]
    for i in range(n):
        _, info = U.decode_step(dims, p, cache, q[:, i], k[:, i], v[:, i], x[:, i], tau)
        for it in info:
            assert np.all(it["A"] <= 0.0)
        for s in range(dims.B * dims.H_kv):
            old = prev[s]
            cur = cache.lam[s][: old.size]
            assert np.all(cur <= old)
            assert not np.any((old < tau) & (cur >= tau))
            prev[s] = cache.lam[s].copy()


# ---------------------------------------------------------------------------
# P7 / P13 / P14: identities between paths
# ---------------------------------------------------------------------------
def _run_decode(dims, p, q, k, v, x, log_p, compact_every=0):
    cache = _fresh(dims)
    ys = []
    for i in range(q.shape[1]):
        y, _ = U.decode_step(dims, p, cache, q[:, i], k[:, i], v[:, i], x[:, i], log_p)
        ys.append(y)
        if compact_every and (i + 1) % compact_every == 0:
            U.compact(cache, log_p)
    return np.stack(ys, axis=1), cache


def test_P7_decode_equals_dense_threshold_attention():
    """Decode at p equals O7 with live_i = {j <= i: Lambda_ij >= tau} (sections 4.2 and 3)."""
    dims = _dims(H_q=2, H_kv=1, d=8, D=5)
    rng = RNG(11)
    p = _params(dims, rng, gate_scale=2.0)
    n = 36
    q, k, v, x = _tokens(dims, n, rng)
    tau = math.log(0.15)
    yd, _ = _run_decode(dims, p, q, k, v, x, tau, compact_every=3)
    qt, kt = _preprocessed(dims, p, q, k, x)
    z = x[0] @ p.W_dec + p.b_dec
    lq, lk, lb = U.log_sigmoid(z[:, 0]), U.log_sigmoid(z[:, 1]), U.log_sigmoid(z[:, 2])
    Lam = U.dense_logbias(dims.terms, kt[:, 0], lq, lk, lb)
    n_dead = 0
    for i in range(n):
        live = Lam[i, : i + 1] >= tau
        n_dead += int((~live).sum())
        e = dims.scale * (kt[: i + 1, 0] @ qt[i].T).T + Lam[i, : i + 1]
        e = np.where(live[None, :], e, -np.inf)
        w = np.exp(e - e.max(axis=1, keepdims=True))
        o = (w / w.sum(axis=1, keepdims=True)) @ v[0, : i + 1, 0]
        np.testing.assert_allclose(yd[0, i], o, rtol=1e-11, atol=1e-12)
    assert n_dead > 0  # the threshold actually bit
    # and p = 0 decode is the prefill
    yp = U.prefill(dims, p, _fresh(dims), q, k, v, x)
    y0, _ = _run_decode(dims, p, q, k, v, x, -math.inf)
    np.testing.assert_allclose(y0, yp, rtol=0, atol=0)


def test_P13_chunked_prefill_equals_one_shot():
    dims = _dims(B=2, H_q=4, H_kv=2, d=8)
    rng = RNG(12)
    p = _params(dims, rng, gamma_one=False)
    n = 20
    q, k, v, x = _tokens(dims, n, rng)
    c1 = _fresh(dims)
    y1 = U.prefill(dims, p, c1, q, k, v, x)
    c2 = _fresh(dims)
    ya = U.prefill(dims, p, c2, q[:, :7], k[:, :7], v[:, :7], x[:, :7])
    yb = U.prefill(dims, p, c2, q[:, 7:], k[:, 7:], v[:, 7:], x[:, 7:])
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y1, rtol=1e-13, atol=1e-14)
    for s in range(4):
        np.testing.assert_allclose(c2.lam[s], c1.lam[s], rtol=1e-13, atol=1e-14)


def test_P14_lazy_compaction_equals_eager():
    dims = _dims(B=2, H_q=4, H_kv=2, d=8, D=5)
    rng = RNG(13)
    p = _params(dims, rng, gate_scale=2.0, gamma_one=False)
    n = 30
    q, k, v, x = _tokens(dims, n, rng)
    tau = math.log(0.15)
    ye, ce = _run_decode(dims, p, q, k, v, x, tau, compact_every=1)
    yl, cl = _run_decode(dims, p, q, k, v, x, tau, compact_every=7)
    yn, cn = _run_decode(dims, p, q, k, v, x, tau, compact_every=0)
    np.testing.assert_allclose(yl, ye, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(yn, ye, rtol=1e-13, atol=1e-14)
    U.compact(cl, tau)
    U.compact(cn, tau)
    for s in range(4):
        np.testing.assert_array_equal(cl.K[s], ce.K[s])
        np.testing.assert_array_equal(cn.K[s], ce.K[s])
        np.testing.assert_allclose(cn.lam[s], ce.lam[s], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# P8: brute force in mpmath on a tiny case
# ---------------------------------------------------------------------------
def test_P8_brute_force_mpmath():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    dims = _dims(H_q=2, H_kv=1, d=4, D=3, r=2)
    rng = RNG(14)
    p = _params(dims, rng, gamma_one=False)
    n = 9
    q, k, v, x = _tokens(dims, n, rng)
    cache = _fresh(dims)
    y = U.prefill(dims, p, cache, q, k, v, x)

    d, half, G = dims.d, dims.d // 2, dims.G
    M = lambda a: [mp.mpf(float(t)) for t in a]

    def rot(vec, pos):
        out = [None] * d
        for i in range(half):
            w = mp.power(mp.mpf(dims.rope_base), -mp.mpf(2 * i) / d)
            c, s = mp.cos(pos * w), mp.sin(pos * w)
            out[i] = vec[i] * c - vec[i + half] * s
            out[i + half] = vec[i + half] * c + vec[i] * s
        return out

    def lsig(zv):
        return -mp.log(1 + mp.exp(-zv))

    keys, qs, lq, lk, lb, gam = [], [], [], [], [], []
    for t in range(n):
        kk = M(k[0, t, 0])
        nrm = mp.sqrt(sum(c * c for c in kk))
        keys.append(rot([c / nrm for c in kk], t))
        qs.append([rot(M(q[0, t, a]), t) for a in range(dims.H_q)])
        xv = M(x[0, t])
        z = [sum(xv[i] * mp.mpf(float(p.W_dec[i, c])) for i in range(dims.D)) + mp.mpf(float(p.b_dec[c])) for c in range(3)]
        lq.append(lsig(z[0]))
        lk.append(lsig(z[1]))
        lb.append(lsig(z[2]))
        u = [sum(xv[i] * mp.mpf(float(p.W_dn[i, c])) for i in range(dims.D)) for c in range(dims.r)]
        g = [sum(u[c] * mp.mpf(float(p.W_up[c, o])) for c in range(dims.r)) + mp.mpf(float(p.b_up[o])) for o in range(dims.H_q * d)]
        gam.append([1 / (1 + mp.exp(-gv)) for gv in g])

    def A(t, j):
        s = sum(keys[t][c] * keys[j][c] for c in range(d))
        lam = (lq[t] + lk[j] + lb[t] + mp.log(min(s * s, mp.mpf(1)))) / 3
        return mp.log(1 - mp.exp(lam))

    for i in range(n):
        Lam = [sum((A(t, j) for t in range(j + 1, i + 1)), mp.mpf(0)) for j in range(i + 1)]
        for a in range(dims.H_q):
            e = [mp.mpf(dims.scale) * sum(qs[i][a][c] * keys[j][c] for c in range(d)) + Lam[j] for j in range(i + 1)]
            w = [mp.exp(ev) for ev in e]
            Z = sum(w)
            for c in range(d):
                o = sum(w[j] * mp.mpf(float(v[0, j, 0, c])) for j in range(i + 1)) / Z
                ref = gam[i][a * d + c] * o
                assert abs(y[0, i, a, c] - float(ref)) <= 1e-12
        if i == n - 1:
            for j in range(n):
                assert abs(cache.lam[0][j] - float(Lam[j])) <= 1e-12


# ---------------------------------------------------------------------------
# P11 / P12 / P15: invariants
# ---------------------------------------------------------------------------
def test_P11_permutation_invariance():
    dims = _dims(H_q=3, H_kv=1, d=8, D=5)
    rng = RNG(15)
    p = _params(dims, rng, gamma_one=False)
    n = 18
    q, k, v, x = _tokens(dims, n, rng)
    cache = _fresh(dims)
    U.prefill(dims, p, cache, q[:, :-1], k[:, :-1], v[:, :-1], x[:, :-1])
    perm = rng.permutation(cache.lam[0].size)
    c2 = cache.copy()
    for name in ("K", "V", "lam", "lk"):
        getattr(c2, name)[0] = getattr(c2, name)[0][perm]
    tau = math.log(0.05)
    y1, _ = U.decode_step(dims, p, cache, q[:, -1], k[:, -1], v[:, -1], x[:, -1], tau)
    y2, _ = U.decode_step(dims, p, c2, q[:, -1], k[:, -1], v[:, -1], x[:, -1], tau)
    np.testing.assert_allclose(y2, y1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(c2.lam[0][:-1], cache.lam[0][:-1][perm], rtol=1e-14, atol=1e-15)


def test_P12_mha_replication_equals_gqa():
    G, H_kv = 2, 2
    dims = _dims(B=1, H_q=G * H_kv, H_kv=H_kv, d=8, D=5)
    rng = RNG(16)
    p = _params(dims, rng, gamma_one=False)
    n = 14
    q, k, v, x = _tokens(dims, n, rng)
    y = U.prefill(dims, p, _fresh(dims), q, k, v, x)
    md = _dims(B=1, H_q=G * H_kv, H_kv=G * H_kv, d=8, D=5)
    rep = np.arange(G * H_kv) // G  # MHA head a uses GQA KV head a // G
    cols = np.concatenate([m * H_kv + rep for m in range(3)])
    mp_ = U.Params(W_dec=p.W_dec[:, cols], b_dec=p.b_dec[cols], W_dn=p.W_dn, W_up=p.W_up, b_up=p.b_up)
    ym = U.prefill(md, mp_, _fresh(md), q, k[:, :, rep], v[:, :, rep], x)
    np.testing.assert_allclose(ym, y, rtol=1e-13, atol=1e-14)


def test_P15_rope_relative_position():
    rng = RNG(17)
    d = 16
    a, b = rng.normal(size=d), rng.normal(size=d)
    for m, n in [(3, 1), (100, 98), (33000, 32998), (7, 5)]:
        val = U.rope(a, m, 10000.0) @ U.rope(b, n, 10000.0)
        ref = U.rope(a, 2, 10000.0) @ U.rope(b, 0, 10000.0)
        assert abs(val - ref) < 1e-9
    # a rotation keeps the norm (keys stay unit after O1 + O2)
    kk = U.rope(U.l2_normalize(rng.normal(size=(5, d))), np.arange(5) * 1000, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(kk, axis=1), 1.0, atol=1e-14)


def test_dense_logbias_matches_recurrence():
    """The column-sum builder of O5 agrees with the decode-style row recurrence."""
    dims = _dims(H_q=2, H_kv=1, d=8, D=5, bf16=True)
    rng = RNG(18)
    p = _params(dims, rng)
    n = 25
    q, k, v, x = _tokens(dims, n, rng)
    cache = _fresh(dims)
    U.prefill(dims, p, cache, q, k, v, x)
    qt, kt = _preprocessed(dims, p, q, k, x)
    z = x[0] @ p.W_dec + p.b_dec
    Lam = U.dense_logbias(dims.terms, kt[:, 0], U.log_sigmoid(z[:, 0]), U.log_sigmoid(z[:, 1]), U.log_sigmoid(z[:, 2]), rows=[n - 1, 5])
    np.testing.assert_allclose(Lam[0], cache.lam[0], rtol=1e-13, atol=1e-14)
    assert np.all(np.isneginf(Lam[1, 6:]))
    # a row asked for twice is filled twice (the sampled full-size checks repeat the last row)
    rep = U.dense_logbias(dims.terms, kt[:, 0], U.log_sigmoid(z[:, 0]), U.log_sigmoid(z[:, 1]),
                          U.log_sigmoid(z[:, 2]), rows=[n - 1, 3, n - 1])
    np.testing.assert_array_equal(rep[0], rep[2])
    np.testing.assert_array_equal(rep[0], Lam[0])


def test_overflow_sets_status_and_skips_append():
    dims = _dims(H_q=2, H_kv=1, d=8)
    rng = RNG(19)
    p = _params(dims, rng)
    q, k, v, x = _tokens(dims, 4, rng)
    cache = _fresh(dims, cap=3)
    for i in range(4):
        y, _ = U.decode_step(dims, p, cache, q[:, i], k[:, i], v[:, i], x[:, i], -math.inf)
    assert cache.status & 1
    assert cache.lam[0].size == 3
    assert cache.next_pos[0] == 4


# ---------------------------------------------------------------------------
# R26: Qwen3-style normalized queries and keys (paperlayer.ai summary,
# Appendix E ablations) as an RMS normalisation over the head dimension
# ---------------------------------------------------------------------------
def test_qk_rmsnorm_worked_example():
    """x = (3, 4): mean square 12.5, so x / sqrt(12.5) = (0.8485..., 1.1313...); weights (1, 2)."""
    y = U.qk_rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), eps=0.0)
    r = math.sqrt(12.5)
    assert np.allclose(y, [3.0 / r, 8.0 / r], rtol=0, atol=1e-15)


def test_qk_rmsnorm_matches_torch_rms_norm():
    """torch's RMSNorm in fp64, weights and eps included, on [B, n, H, d] heads."""
    rng = RNG(7)
    x = rng.normal(0, 3, (2, 5, 4, 64))
    w = rng.normal(1, 0.2, 64)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (64,), weight=torch.tensor(w), eps=1e-6).numpy()
    assert np.allclose(U.qk_rmsnorm(x, w), ref, rtol=1e-13, atol=1e-13)


def test_qk_rmsnorm_invariants():
    """Unit mean square with unit weights and eps = 0; invariant to a positive scale of
    the head vector; heads are normalised independently."""
    rng = RNG(8)
    x = rng.normal(0, 1, (6, 3, 128))
    one = np.ones(128)
    y = U.qk_rmsnorm(x, one, eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-13)
    assert np.allclose(U.qk_rmsnorm(7.5 * x, one, eps=0.0), y, atol=1e-13)
    x2 = x.copy()
    x2[:, 1] *= 100.0
    y2 = U.qk_rmsnorm(x2, one, eps=0.0)
    assert np.allclose(y2[:, 0], y[:, 0]) and np.allclose(y2[:, 2], y[:, 2])


def test_P_varlen_prefill_is_each_sequence_on_its_own():
    """R31 (per-sequence, per-KV-head caches: paperlayer.ai section 4.2): a packed
    variable-length prefill gives, for each sequence, O5-O7 over that sequence's
    own tokens alone (brute force: the dense bias and softmax written out), leaves
    an empty sequence untouched, and advances each position by its own count."""
    dims = _dims(B=3, H_q=4, H_kv=2, d=8, D=5)
    rng = RNG(31)
    p = _params(dims, rng, gate_scale=2.0)  # gamma = 1: y is the attention output
    lens = [5, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q = rng.normal(0, 1, (T, dims.H_q, dims.d))
    k = rng.normal(0, 1, (T, dims.H_kv, dims.d))
    v = rng.normal(0, 1, (T, dims.H_kv, dims.d))
    x = rng.normal(0, 1, (T, dims.D))
    cache = _fresh(dims)
    cache.next_pos[:] = [3, 7, 0]
    y = U.prefill_varlen(dims, p, cache, q, k, v, x, cu)
    G = dims.G
    for b, n in enumerate(lens):
        r = slice(cu[b], cu[b + 1])
        one = _dims(B=1, H_q=4, H_kv=2, d=8, D=5)
        pos0 = [3, 7, 0][b]
        assert cache.next_pos[b] == pos0 + n
        for h in range(dims.H_kv):
            assert cache.lam[b * dims.H_kv + h].shape[0] == n
        if n == 0:
            continue
        qt, kt = _preprocessed(one, p, q[None, r], k[None, r], x[None, r], pos0=pos0)
        z = x[r] @ p.W_dec + p.b_dec
        for h in range(dims.H_kv):
            lq, lk, lb = (U.log_sigmoid(z[:, c * dims.H_kv + h]) for c in range(3))
            Lam = U.dense_logbias(dims.terms, kt[:, h], lq, lk, lb)
            np.testing.assert_allclose(cache.lam[b * dims.H_kv + h], Lam[n - 1], rtol=1e-12, atol=1e-13)
            for i in range(n):
                e = dims.scale * (kt[: i + 1, h] @ qt[i, h * G:(h + 1) * G].T).T + Lam[i, : i + 1]
                w = np.exp(e - e.max(axis=1, keepdims=True))
                o = (w / w.sum(axis=1, keepdims=True)) @ v[r][: i + 1, h]
                np.testing.assert_allclose(y[cu[b] + i, h * G:(h + 1) * G], o, rtol=1e-11, atol=1e-12)


def test_P_varlen_equal_lengths_is_batched_prefill():
    dims = _dims(B=2, H_q=4, H_kv=2, d=8)
    rng = RNG(32)
    p = _params(dims, rng, gamma_one=False)
    n = 6
    q, k, v, x = _tokens(dims, n, rng)
    c1, c2 = _fresh(dims), _fresh(dims)
    y1 = U.prefill(dims, p, c1, q, k, v, x)
    flat = lambda a: a.reshape((-1,) + a.shape[2:])
    y2 = U.prefill_varlen(dims, p, c2, flat(q), flat(k), flat(v), flat(x), [0, n, 2 * n])
    np.testing.assert_array_equal(y2.reshape(y1.shape), y1)
    for s in range(4):
        np.testing.assert_array_equal(c2.lam[s], c1.lam[s])
