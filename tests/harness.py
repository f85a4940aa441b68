"""Shared parity machinery: the same seeded inputs go to the oracle and to the
HIP path (through the C ABI), and outputs are compared with the tolerances
of the spec: y max-abs 1e-2 (bf16) / 1e-4 (fp32); log-biases
|d| <= 1e-4 * max(|oracle|, 1); keep masks identical except entries within
1e-4 of log p, where the oracle adopts the GPU's value; compaction exact.
"""

from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

import oracle as U
from ua_inputs import LayerConfig, Weights, CacheInit, make_cache, make_step_inputs, make_weights

BORDER = 1e-4


def y_tol(cfg: LayerConfig) -> float:
    return 1e-2 if cfg.bf16 else 1e-4


def oracle_dims(cfg: LayerConfig, terms: int = U.TERMS_ALL) -> U.Dims:
    return U.Dims(B=cfg.B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, D=cfg.D, r=cfg.r, terms=terms, rope_base=10000.0,
                  cache_bf16=cfg.bf16)


def oracle_params(w: Weights) -> U.Params:
    f = lambda a: np.asarray(a, np.float64)
    return U.Params(W_dec=f(w.W_dec), b_dec=f(w.b_dec), W_dn=f(w.W_dn), W_up=f(w.W_up), b_up=f(w.b_up))


def oracle_cache(cfg: LayerConfig, c: CacheInit) -> U.RefCache:
    S = cfg.B * cfg.H_kv
    rc = U.RefCache.empty(oracle_dims(cfg), c.seg_cap, c.next_pos)
    for s in range(S):
        o, n = int(c.seg_off[s]), int(c.seg_len[s])
        rc.K[s] = c.K[o : o + n].astype(np.float64)
        rc.V[s] = c.V[o : o + n].astype(np.float64)
        rc.lam[s] = c.lam[o : o + n].astype(np.float64)
        rc.lk[s] = c.lk[o : o + n].astype(np.float64)
    return rc


def device_layer(cfg: LayerConfig, w: Weights, c: CacheInit, terms: int = 7, max_tokens: int = 1, y_bf16=False):
    from kv_cache_pruning_amd.layer import layer_from_arrays

    return layer_from_arrays(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, cfg.D, cfg.r, cfg.bf16, w, c, terms=terms,
                             max_tokens=max_tokens, y_bf16=y_bf16)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (for the stored-key check)."""
    ax = np.maximum(np.abs(x), 2.0**-126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


@dataclass
class StepReport:
    step: int
    y_err: float
    lam_err: float
    n_border: int
    n_updated: int
    n_dead: int
    lam_err_strict: float = 0.0  # |d| / max(|oracle|, 1e-6): relative down to tiny biases (reported)


@dataclass
class DecodeRun:
    reports: List[StepReport] = field(default_factory=list)

    @property
    def max_y_err(self):
        return max(r.y_err for r in self.reports)

    @property
    def max_lam_err(self):
        return max(r.lam_err for r in self.reports)

    @property
    def max_lam_err_strict(self):
        return max(r.lam_err_strict for r in self.reports)

    @property
    def borderline(self):
        return sum(r.n_border for r in self.reports)


def gpu_state(layer):
    """Copy the device cache back to numpy (fp64 values)."""
    c = layer.cache
    return dict(  # K, V as fp32 (exact for bf16 and fp32 caches)
        K=c.K.float().cpu().numpy(),
        V=c.V.float().cpu().numpy(),
        lam=c.logbias.cpu().numpy().astype(np.float64),
        lk=c.kgate.cpu().numpy().astype(np.float64),
        seg_off=c.seg_off.cpu().numpy(),
        seg_len=c.seg_len.cpu().numpy(),
        next_pos=c.next_pos.cpu().numpy(),
        status=int(c.status.cpu().numpy()[0]),
    )


def run_decode_parity(cfg: LayerConfig, steps: int, log_p: float, compact_every: int = 1, terms: int = 7,
                      seed: int = 0, check_kept: bool = True) -> DecodeRun:
    """Decode `steps` steps on the GPU and in the oracle, comparing every step."""
    import torch

    w = make_weights(cfg, seed)
    c = make_cache(cfg, w, seed)
    layer = device_layer(cfg, w, c, terms=terms)
    od, op = oracle_dims(cfg, terms), oracle_params(w)
    oc = oracle_cache(cfg, c)
    S = cfg.B * cfg.H_kv
    run = DecodeRun()
    kept_buf = torch.full((layer.cache.total_slots,), -1, dtype=torch.int32, device="cuda")
    for step in range(steps):
        inp = make_step_inputs(cfg, step, 1, seed)
        q, k, v, x = inp.q[:, 0], inp.k[:, 0], inp.v[:, 0], inp.x[:, 0]
        len_before = layer.cache.seg_len.cpu().numpy().copy()
        y_gpu, _ = layer.decode_step(q, k, v, x, log_p)
        torch.cuda.synchronize()
        g = gpu_state(layer)
        y_gpu = y_gpu.float().cpu().numpy().astype(np.float64)
        # stored new keys (R17): within one bf16 ulp (fp32: 1e-6 relative) of the oracle's own
        k_gpu = np.zeros((cfg.B, cfg.H_kv, cfg.d))
        for s in range(S):
            b, h = divmod(s, cfg.H_kv)
            if len_before[s] < int(c.seg_cap[s]):
                k_gpu[b, h] = g["K"][int(g["seg_off"][s]) + len_before[s]]
            else:
                k_gpu[b, h] = np.nan
        pos = oc.next_pos.copy()
        k_or = np.stack([U.round_cache(od, U.rope(U.l2_normalize(np.asarray(k[b], np.float64)),
                                                    np.full(cfg.H_kv, pos[b]), od.rope_base)) for b in range(cfg.B)])
        have = ~np.isnan(k_gpu[..., 0])
        tol = np.maximum(ulp_bf16(k_or), 2e-7) if cfg.bf16 else 2e-6
        bad = (np.abs(k_gpu - k_or) > tol * 1.0001) & have[..., None]
        assert not bad.any(), f"step {step}: stored key off by more than one ulp"
        k_use = np.where(have[..., None], k_gpu, k_or)

        # oracle step, adopting the GPU's decision for borderline entries
        tau = log_p
        border_log = {}

        def decide(s, lam_new, idx):
            o = int(g["seg_off"][s])
            lam_g = g["lam"][o + idx]
            live_o = lam_new >= tau
            live_g = np.float32(lam_g) >= np.float32(tau)  # the kernel's own test, in fp32
            border = np.abs(lam_new - tau) <= BORDER
            border_log[s] = (idx[border], lam_g[border], live_g[border])
            mismatch = (live_o != live_g) & ~border
            assert not mismatch.any(), f"step {step} seg {s}: keep mask differs away from the threshold"
            return np.where(border, live_g, live_o)

        y_or, info = U.decode_step(od, op, oc, q, k, v, x, log_p, decide=decide, k_override=k_use)
        # adopt borderline GPU values so both trajectories continue from the same state
        nb = 0
        for s, (bidx, lamg, liveg) in border_log.items():
            # the GPU's value, on the GPU's side of tau: fp32(log p) lies a few 1e-8 below log p,
            # so a kept fp32 bias may sit just under the fp64 threshold
            oc.lam[s][bidx] = np.where(liveg, np.maximum(lamg, tau), np.minimum(lamg, np.nextafter(tau, -np.inf)))
            nb += len(bidx)
        y_err = float(np.max(np.abs(y_gpu - y_or)))
        lam_err = 0.0
        lam_strict = 0.0
        n_upd = 0
        n_dead = 0
        for it in info:
            s = it["seg"]
            idx = it["updated_idx"]
            o = int(g["seg_off"][s])
            lo = oc.lam[s][idx]
            lg = g["lam"][o + idx]
            fin = np.isfinite(lo)
            assert np.array_equal(np.isneginf(lo), np.isneginf(lg)), f"step {step}: -inf pattern differs"
            if fin.any():
                lam_err = max(lam_err, _maxrel(lg[fin], lo[fin]))
                lam_strict = max(lam_strict, _maxrel(lg[fin], lo[fin], 1e-6))
            n_upd += idx.size
            n_dead += int((~it["live"]).sum())
        # lengths, positions, status
        assert np.array_equal(g["seg_len"], oc.lengths()), f"step {step}: segment lengths differ"
        assert np.array_equal(g["next_pos"], oc.next_pos), f"step {step}: positions differ"
        assert g["status"] == oc.status, f"step {step}: status differs"
        run.reports.append(StepReport(step, y_err, lam_err, nb, n_upd, n_dead, lam_strict))
        if steps >= 64 and (step + 1) % 32 == 0:
            print(f"    step {step + 1}/{steps}: max |dy| {run.max_y_err:.2e}, max rel dLambda "
                  f"{run.max_lam_err:.2e}", flush=True)
        assert y_err <= y_tol(cfg), f"step {step}: y max-abs error {y_err:.3e}"
        assert lam_err <= 1e-4, f"step {step}: log-bias error {lam_err:.3e}"

        if compact_every and (step + 1) % compact_every == 0:
            before = gpu_state(layer)
            kept_buf.fill_(-1)
            layer.compact(log_p, kept_buf if check_kept else None)
            torch.cuda.synchronize()
            after = gpu_state(layer)
            kept_or = U.compact(oc, log_p)
            kb = kept_buf.cpu().numpy()
            for s in range(S):
                o = int(after["seg_off"][s])
                n = int(after["seg_len"][s])
                assert n == kept_or[s].size, f"step {step} seg {s}: compacted length differs"
                if check_kept:
                    assert np.array_equal(kb[o : o + n], kept_or[s]), f"step {step} seg {s}: kept index list differs"
                src = o + kept_or[s]
                for name in ("K", "V", "lam", "lk"):
                    assert np.array_equal(after[name][o : o + n], before[name][src]), \
                        f"step {step} seg {s}: moved {name} rows differ"
    return run


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def _maxabs(a, b) -> float:
    """max |a - b|; inf if either side holds a NaN (so a NaN can never pass)."""
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    return float("inf") if np.isnan(d).any() else float(np.max(d, initial=0.0))


def _maxrel(a, b, floor: float = 1.0) -> float:
    """max |a - b| / max(|b|, floor); inf on NaN."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    d = np.abs(a - b) / np.maximum(np.abs(b), floor)
    return float("inf") if np.isnan(d).any() else float(np.max(d, initial=0.0))


def _check_new_keys(cfg, od, k_in, pos0, k_gpu):
    """Stored new keys (R17): within one bf16 ulp of the oracle's own rounding.

    k_in [B, n, H_kv, d] raw keys, pos0 [B] first positions, k_gpu [B, n, H_kv, d].
    """
    B, n = k_in.shape[0], k_in.shape[1]
    k_or = np.empty_like(k_gpu)
    for b in range(B):
        for t in range(n):
            k_or[b, t] = U.round_cache(od, U.rope(U.l2_normalize(np.asarray(k_in[b, t], np.float64)),
                                                  np.full(cfg.H_kv, pos0[b] + t), od.rope_base))
    tol = np.maximum(ulp_bf16(k_or), 2e-7) if cfg.bf16 else 2e-6
    bad = np.abs(k_gpu - k_or) > tol * 1.0001
    assert not bad.any(), f"stored prefill key off by more than one ulp ({int(bad.sum())} elements)"


def _stored_new(g, c_off, len_before, cfg, n, field):
    """Rows [len_before, len_before + n) of every segment as [B, n, H_kv, ...]."""
    out = []
    for b in range(cfg.B):
        rows = []
        for h in range(cfg.H_kv):
            s = b * cfg.H_kv + h
            o = int(c_off[s]) + int(len_before[s])
            rows.append(g[field][o : o + n])
        out.append(np.stack(rows, axis=1))
    return np.stack(out)


def run_prefill_parity(cfg: LayerConfig, calls: Optional[int] = None, terms: int = 7, seed: int = 0,
                       y_bf16: bool = False) -> dict:
    """Chunked prefill on the GPU and in the oracle, compared after every call.

    ``cfg.chunk`` tokens per call, ``calls`` calls (default n_total / chunk).
    Compares y (max-abs), every cached log-bias (relative 1e-4), the stored
    keys (one ulp), values (exact), key gates, lengths, positions and status.
    """
    import torch

    calls = calls if calls is not None else cfg.n_total // cfg.chunk
    n = cfg.chunk
    w = make_weights(cfg, seed)
    c = make_cache(cfg, w, seed)
    layer = device_layer(cfg, w, c, terms=terms, max_tokens=n, y_bf16=y_bf16)
    od, op = oracle_dims(cfg, terms), oracle_params(w)
    oc = oracle_cache(cfg, c)
    S = cfg.B * cfg.H_kv
    rep = {"y_err": 0.0, "lam_err": 0.0, "lk_err": 0.0, "calls": calls}
    for call in range(calls):
        inp = make_step_inputs(cfg, call, n, seed)
        len_before = layer.cache.seg_len.cpu().numpy().copy()
        pos0 = layer.cache.next_pos.cpu().numpy().copy()
        y_gpu, _ = layer.prefill(inp.q, inp.k, inp.v, inp.x)
        torch.cuda.synchronize()
        g = gpu_state(layer)
        k_gpu = _stored_new(g, c.seg_off, len_before, cfg, n, "K")
        _check_new_keys(cfg, od, inp.k, pos0, k_gpu)
        v_gpu = _stored_new(g, c.seg_off, len_before, cfg, n, "V")
        assert np.array_equal(v_gpu, inp.v.astype(np.float64)), f"call {call}: appended values differ"
        y_or = U.prefill(od, op, oc, inp.q, inp.k, inp.v, inp.x, k_override=k_gpu)
        y_err = _maxabs(y_gpu.float().cpu().numpy(), y_or)
        lam_err = 0.0
        lk_err = 0.0
        for s in range(S):
            o, m = int(c.seg_off[s]), int(g["seg_len"][s])
            assert m == oc.lam[s].size, f"call {call} seg {s}: length differs"
            lg, lo = g["lam"][o : o + m], oc.lam[s]
            assert np.array_equal(np.isneginf(lg), np.isneginf(lo)), f"call {call} seg {s}: -inf pattern differs"
            fin = np.isfinite(lo)
            lam_err = max(lam_err, _maxrel(lg[fin], lo[fin]))
            lk_err = max(lk_err, _maxrel(g["lk"][o : o + m], oc.lk[s]))
        assert np.array_equal(g["next_pos"], oc.next_pos), f"call {call}: positions differ"
        assert g["status"] == 0, f"call {call}: status {g['status']}"
        rep["y_err"] = max(rep["y_err"], y_err)
        rep["lam_err"] = max(rep["lam_err"], lam_err)
        rep["lk_err"] = max(rep["lk_err"], lk_err)
        assert y_err <= y_tol(cfg), f"call {call}: y max-abs error {y_err:.3e}"
        assert lam_err <= 1e-4, f"call {call}: log-bias error {lam_err:.3e}"
        assert lk_err <= 1e-5, f"call {call}: key-gate error {lk_err:.3e}"
    return rep


def run_prefill_full(cfg: LayerConfig, rows_per_call: int = 16, log_p: Optional[float] = None, seed: int = 0,
                     terms: int = 7, workers: int = 8, segments=None) -> dict:
    """Full-size prefill from an empty cache, then one eviction at log_p.

    Runs every call of ``cfg`` (chunk tokens each) on the GPU in the library's
    normal launch configuration.  For every segment (or those given), the
    oracle's dense definitions give y at ``rows_per_call`` seeded rows of
    every call (and the last token) and the final log-bias of every key; the
    stored keys and key gates are checked for all tokens.  Then ua_compact at
    log_p: the kept-index lists must equal np.flatnonzero of the GPU's final
    mask exactly, with moved rows bit-identical, and that mask must equal the
    oracle's except entries within 1e-4 of log p (counted).
    """
    import concurrent.futures as cf
    import multiprocessing as mp

    import torch

    n = cfg.chunk
    calls = cfg.n_total // n
    N = n * calls
    w = make_weights(cfg, seed)
    c = make_cache(cfg, w, seed)
    assert int(np.max(c.seg_len)) == 0, "the full check starts from an empty cache"
    layer = device_layer(cfg, w, c, terms=terms, max_tokens=n)
    od, op = oracle_dims(cfg, terms), oracle_params(w)
    S = cfg.B * cfg.H_kv
    G = cfg.H_q // cfg.H_kv
    segments = list(range(S)) if segments is None else list(segments)
    rng = np.random.default_rng(1234)
    q_all = np.zeros((cfg.B, N, cfg.H_q, cfg.d), np.float32)
    k_all = np.zeros((cfg.B, N, cfg.H_kv, cfg.d), np.float32)
    x_all = np.zeros((cfg.B, N, cfg.D), np.float32)
    rows, y_rows = [], []
    for call in range(calls):
        inp = make_step_inputs(cfg, call, n, seed)
        y, _ = layer.prefill(inp.q, inp.k, inp.v, inp.x)
        pick = set(int(t) for t in rng.choice(n, rows_per_call, replace=False))
        if call == calls - 1:
            pick.add(n - 1)
        pick = sorted(pick)
        y_rows.append(y[:, pick].float().cpu().numpy().astype(np.float64))
        rows.extend(call * n + t for t in pick)
        q_all[:, call * n : (call + 1) * n] = inp.q
        k_all[:, call * n : (call + 1) * n] = inp.k
        x_all[:, call * n : (call + 1) * n] = inp.x
    torch.cuda.synchronize()
    y_gpu = np.concatenate(y_rows, axis=1)  # [B, len(rows), H_q, d]
    g = gpu_state(layer)
    assert g["status"] == 0 and np.all(g["seg_len"] == N)
    rows = np.asarray(rows)
    rep = {"y_err": 0.0, "lam_err": 0.0, "n_rows": int(rows.size) * len(segments), "segments": len(segments)}
    jobs = []
    for s in segments:
        b, h = divmod(s, cfg.H_kv)
        o = int(c.seg_off[s])
        Kt = g["K"][o : o + N].astype(np.float64)
        k_or = U.round_cache(od, U.rope(U.l2_normalize(np.asarray(k_all[b][:, h], np.float64)), np.arange(N),
                                        od.rope_base))
        tol = np.maximum(ulp_bf16(k_or), 2e-7)
        assert not np.any(np.abs(Kt - k_or) > tol * 1.0001), f"seg {s}: stored key off by more than one ulp"
        lq, lk, lb = U.gates(od, op, x_all[b])
        lkg = g["lk"][o : o + N]
        assert np.max(np.abs(lkg - lk[:, h]) / np.maximum(np.abs(lk[:, h]), 1.0)) <= 1e-5, f"seg {s}: key gates"
        V = g["V"][o : o + N].astype(np.float64)
        assert np.all(np.isfinite(Kt)) and np.all(np.isfinite(V)), f"seg {s}: non-finite cache rows"
        q_rows = q_all[b][rows, h * G : (h + 1) * G].astype(np.float64)
        gam_rows = np.stack([U.output_gate(od, op, x_all[b][i])[h * G : (h + 1) * G] for i in rows])
        jobs.append((terms, Kt, V, lq[:, h], lk[:, h], lb[:, h], q_rows, gam_rows, rows, od.scale, od.rope_base))
    from tests.oracle_worker import segment_prefill_oracle

    print(f"    GPU calls done; oracle on {len(jobs)} segments in {min(workers, len(jobs))} processes", flush=True)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"  # one BLAS thread per worker process
    ctx = mp.get_context("spawn")
    results = [None] * len(jobs)
    with cf.ProcessPoolExecutor(max_workers=min(workers, len(jobs)), mp_context=ctx) as ex:
        futs = {ex.submit(segment_prefill_oracle, j): i for i, j in enumerate(jobs)}
        for n_done, f in enumerate(cf.as_completed(futs)):
            results[futs[f]] = f.result()
            print(f"    oracle segment {n_done + 1}/{len(jobs)} done", flush=True)
    lam_final = {}
    for s, (lo, ys) in zip(segments, results):
        b, h = divmod(s, cfg.H_kv)
        o = int(c.seg_off[s])
        lam_fin = g["lam"][o : o + N]
        fin = np.isfinite(lo)
        assert np.array_equal(np.isneginf(lam_fin), np.isneginf(lo)), f"seg {s}: -inf pattern differs"
        rep["lam_err"] = max(rep["lam_err"], _maxrel(lam_fin[fin], lo[fin]))
        assert np.all(np.isfinite(ys)), f"seg {s}: oracle output not finite"
        rep["y_err"] = max(rep["y_err"], _maxabs(y_gpu[b, :, h * G : (h + 1) * G], ys))
        lam_final[s] = lo
    assert rep["y_err"] <= y_tol(cfg), f"sampled y max-abs error {rep['y_err']:.3e}"
    assert rep["lam_err"] <= 1e-4, f"final log-bias error {rep['lam_err']:.3e}"
    if log_p is None:
        return rep
    # ---- eviction at log_p over the whole cache
    before = gpu_state(layer)
    kept_buf = torch.full((layer.cache.total_slots,), -1, dtype=torch.int32, device="cuda")
    layer.compact(log_p, kept_buf)
    torch.cuda.synchronize()
    after = gpu_state(layer)
    kb = kept_buf.cpu().numpy()
    assert after["status"] == 0
    rep["kept"] = 0
    rep["borderline"] = 0
    for s in range(S):
        o = int(c.seg_off[s])
        lam_g = before["lam"][o : o + N]
        keep = np.flatnonzero(lam_g >= np.float32(log_p))
        m = int(after["seg_len"][s])
        assert m == keep.size, f"seg {s}: {m} entries kept, the mask has {keep.size}"
        assert np.array_equal(kb[o : o + m], keep), f"seg {s}: kept list is not flatnonzero of the mask"
        for name in ("K", "V", "lam", "lk"):
            assert np.array_equal(after[name][o : o + m], before[name][o + keep]), f"seg {s}: moved {name} differ"
        rep["kept"] += m
        if s in lam_final:
            lo = lam_final[s]
            live_o, live_g = lo >= log_p, lam_g >= np.float32(log_p)
            border = np.abs(lo - log_p) <= BORDER
            assert not ((live_o != live_g) & ~border).any(), f"seg {s}: keep mask differs away from log p"
            rep["borderline"] += int(border.sum())
    return rep


# ---------------------------------------------------------------------------
# decode step and compaction in one launch
# ---------------------------------------------------------------------------
def run_fused_parity(cfg: LayerConfig, steps: int, log_p: float, terms: int = 7, seed: int = 0) -> DecodeRun:
    """ua_decode_compact_step vs the oracle's decode step followed by compaction.

    Per step: y; the kept-index lists exactly; the surviving rows (K, V) bit
    for bit; log-biases (relative 1e-4), key gates, lengths, positions and
    status.  Entries within 1e-4 of log p take the GPU's keep decision (read
    from its kept list) and, when kept, its log-bias.
    """
    import torch

    w = make_weights(cfg, seed)
    c = make_cache(cfg, w, seed)
    layer = device_layer(cfg, w, c, terms=terms)
    od, op = oracle_dims(cfg, terms), oracle_params(w)
    oc = oracle_cache(cfg, c)
    S = cfg.B * cfg.H_kv
    run = DecodeRun()
    kept_buf = torch.full((layer.cache.total_slots,), -1, dtype=torch.int32, device="cuda")
    tau = log_p
    for step in range(steps):
        inp = make_step_inputs(cfg, step, 1, seed)
        q, k, v, x = inp.q[:, 0], inp.k[:, 0], inp.v[:, 0], inp.x[:, 0]
        len_before = layer.cache.seg_len.cpu().numpy().copy()
        kept_buf.fill_(-1)
        y_gpu, _ = layer.decode_compact_step(q, k, v, x, log_p, kept=kept_buf)
        torch.cuda.synchronize()
        g = gpu_state(layer)
        kb = kept_buf.cpu().numpy()
        y_gpu = y_gpu.float().cpu().numpy().astype(np.float64)
        assert g["status"] == 0, f"step {step}: status {g['status']}"
        # per segment: surviving pre-step indices and where they went
        kept_g, where_g = {}, {}
        k_gpu = np.zeros((cfg.B, cfg.H_kv, cfg.d))
        for s in range(S):
            b, h = divmod(s, cfg.H_kv)
            o, n = int(g["seg_off"][s]), int(g["seg_len"][s])
            kl = kb[o : o + n].astype(np.int64)
            assert n >= 1 and kl[-1] == len_before[s], f"step {step} seg {s}: new entry missing or not last"
            assert np.all(np.diff(kl) > 0), f"step {step} seg {s}: kept list not increasing"
            kept_g[s] = kl
            where_g[s] = {int(j): o + p for p, j in enumerate(kl)}
            k_gpu[b, h] = g["K"][o + n - 1]
        pos = oc.next_pos.copy()
        k_or = np.stack([U.round_cache(od, U.rope(U.l2_normalize(np.asarray(k[b], np.float64)),
                                                    np.full(cfg.H_kv, pos[b]), od.rope_base)) for b in range(cfg.B)])
        tol = np.maximum(ulp_bf16(k_or), 2e-7) if cfg.bf16 else 2e-6
        assert not np.any(np.abs(k_gpu - k_or) > tol * 1.0001), f"step {step}: stored key off by more than one ulp"

        border_fix = {}

        def decide(s, lam_new, idx):
            live_o = lam_new >= tau
            live_g = np.array([int(j) in where_g[s] for j in idx], bool)
            border = np.abs(lam_new - tau) <= BORDER
            assert not ((live_o != live_g) & ~border).any(), f"step {step} seg {s}: keep mask differs away from log p"
            border_fix[s] = (idx[border], live_g[border])
            return np.where(border, live_g, live_o)

        y_or, info = U.decode_step(od, op, oc, q, k, v, x, log_p, decide=decide, k_override=k_gpu)
        nb = 0
        for s, (bidx, bl) in border_fix.items():
            for j, lv in zip(bidx, bl):
                # the GPU's value on the GPU's side of tau (fp32(log p) lies just below log p)
                oc.lam[s][j] = max(g["lam"][where_g[s][int(j)]], tau) if lv else \
                    min(oc.lam[s][j], np.nextafter(tau, -np.inf))
                nb += 1
        kept_or = U.compact(oc, log_p)
        y_err = _maxabs(y_gpu, y_or)
        lam_err = 0.0
        lam_strict = 0.0
        n_dead = 0
        for s in range(S):
            o, n = int(g["seg_off"][s]), int(g["seg_len"][s])
            assert np.array_equal(kept_g[s], kept_or[s]), f"step {step} seg {s}: kept lists differ"
            assert n == oc.lam[s].size
            assert np.array_equal(g["K"][o : o + n], oc.K[s]), f"step {step} seg {s}: K rows differ"
            assert np.array_equal(g["V"][o : o + n], oc.V[s]), f"step {step} seg {s}: V rows differ"
            lg, lo = g["lam"][o : o + n], oc.lam[s]
            assert np.array_equal(np.isneginf(lg), np.isneginf(lo)), f"step {step}: -inf pattern differs"
            fin = np.isfinite(lo)
            lam_err = max(lam_err, _maxrel(lg[fin], lo[fin]))
            lam_strict = max(lam_strict, _maxrel(lg[fin], lo[fin], 1e-6))
            assert _maxrel(g["lk"][o : o + n], oc.lk[s]) <= 1e-5, f"step {step} seg {s}: key gates differ"
            n_dead += int(len_before[s] + 1 - n)
        assert np.array_equal(g["next_pos"], oc.next_pos), f"step {step}: positions differ"
        run.reports.append(StepReport(step, y_err, lam_err, nb, int(np.sum(len_before)), n_dead, lam_strict))
        if steps >= 64 and (step + 1) % 32 == 0:
            print(f"    step {step + 1}/{steps}: max |dy| {run.max_y_err:.2e}, max rel dLambda "
                  f"{run.max_lam_err:.2e}", flush=True)
        assert y_err <= y_tol(cfg), f"step {step}: y max-abs error {y_err:.3e}"
        assert lam_err <= 1e-4, f"step {step}: log-bias error {lam_err:.3e}"
    return run


# ---------------------------------------------------------------------------
# pruned prefill and chunk-boundary eviction
# ---------------------------------------------------------------------------
def _probe_layer(cfg: LayerConfig, w: Weights, c: CacheInit, terms: int, n: int):
    """An empty cache with room for n tokens per segment at the same positions:
    a dense prefill there stores the very key bits the tested call stores."""
    S = cfg.B * cfg.H_kv
    pc = CacheInit(K=np.zeros((S * n, cfg.d), np.float32), V=np.zeros((S * n, cfg.d), np.float32),
                   lam=np.zeros(S * n, np.float32), lk=np.zeros(S * n, np.float32),
                   seg_off=np.arange(S, dtype=np.int64) * n, seg_len=np.zeros(S, np.int32),
                   seg_cap=np.full(S, n, np.int32), next_pos=c.next_pos.copy())
    return device_layer(cfg, w, pc, terms=terms, max_tokens=n), pc


def _compare_cache(layer, oc, cfg, what: str) -> float:
    """Lengths, stored rows and biases of every segment against the oracle."""
    g = gpu_state(layer)
    S = cfg.B * cfg.H_kv
    lam_err = 0.0
    for s in range(S):
        o, m = int(g["seg_off"][s]), int(g["seg_len"][s])
        assert m == oc.lam[s].size, f"{what} seg {s}: {m} entries kept, oracle {oc.lam[s].size}"
        assert np.array_equal(g["K"][o : o + m], oc.K[s]), f"{what} seg {s}: kept keys differ"
        assert np.array_equal(g["V"][o : o + m], oc.V[s]), f"{what} seg {s}: kept values differ"
        lam_err = max(lam_err, _maxrel(g["lam"][o : o + m], oc.lam[s]))
        assert _maxrel(g["lk"][o : o + m], oc.lk[s]) <= 1e-5, f"{what} seg {s}: key gates differ"
    assert np.array_equal(g["next_pos"], oc.next_pos), f"{what}: positions differ"
    assert g["status"] == 0, f"{what}: status {g['status']}"
    return lam_err


def _cache_mismatch(g, oc, cfg, what: str, kept=None, kept_or=None):
    """First difference between the GPU cache state and the oracle's, or None.

    Lengths, kept rows (keys and values bit-exact), log-biases (relative
    1e-4), key gates (1e-5), positions and status; the kept-index lists when
    both are given.  Returns (message or None, max log-bias error).
    """
    S = cfg.B * cfg.H_kv
    lam_err = 0.0
    for s in range(S):
        o, m = int(g["seg_off"][s]), int(g["seg_len"][s])
        if m != oc.lam[s].size:
            return f"{what} seg {s}: {m} entries kept, oracle {oc.lam[s].size}", lam_err
        if kept is not None and not np.array_equal(kept[o : o + m], kept_or[s]):
            return f"{what} seg {s}: kept-index lists differ", lam_err
        if not np.array_equal(g["K"][o : o + m], oc.K[s]):
            return f"{what} seg {s}: kept keys differ", lam_err
        if not np.array_equal(g["V"][o : o + m], oc.V[s]):
            return f"{what} seg {s}: kept values differ", lam_err
        lo, lg = oc.lam[s], g["lam"][o : o + m]
        if not np.array_equal(np.isneginf(lg), np.isneginf(lo)):
            return f"{what} seg {s}: -inf pattern differs", lam_err
        fin = np.isfinite(lo)
        lam_err = max(lam_err, _maxrel(lg[fin], lo[fin]))
        if _maxrel(g["lk"][o : o + m], oc.lk[s]) > 1e-5:
            return f"{what} seg {s}: key gates differ", lam_err
    if not np.array_equal(g["next_pos"], oc.next_pos):
        return f"{what}: positions differ", lam_err
    if g["status"] != 0:
        return f"{what}: status {g['status']}", lam_err
    if lam_err > 1e-4:
        return f"{what}: log-bias error {lam_err:.3e}", lam_err
    return None, lam_err


def _force(lam: np.ndarray, sel: np.ndarray, live: np.ndarray, tau: float):
    """Make the stored biases agree with forced keep decisions: a kept entry
    sits at or above tau, an evicted one strictly below."""
    if sel.size:
        lam[sel[live]] = np.maximum(lam[sel[live]], tau)
        lam[sel[~live]] = np.minimum(lam[sel[~live]], np.nextafter(tau, -np.inf))


def run_pruned_prefill_parity(cfg: LayerConfig, log_p: float, chunked: bool = False, terms: int = 7,
                              seed: int = 0, max_depth: int = 6, max_runs: int = 256) -> dict:
    """ua_prefill_pruned or ua_prefill_chunked on the GPU against the oracle.

    pruned (chunked=False): n_total / chunk calls of `chunk` tokens; each equals
    `chunk` oracle decode steps at log_p (an entry below tau is neither
    attended nor updated again) followed by compaction.
    chunked: one ua_prefill_chunked call over all n_total tokens with chunks of
    `chunk`; it equals, chunk by chunk, the oracle's dense prefill followed by
    compaction at log_p.
    y, the kept entries (keys and values bit-exact, biases relative 1e-4), the
    kept-index lists (pruned) and the lengths are compared after every call.

    A keep decision whose oracle bias lies within 1e-4 of log p may go either
    way on the GPU, and the GPU's per-step decisions are not visible.  Each
    such decision is an event; when the oracle's own decisions do not
    reproduce the GPU's call, the oracle is rerun with events flipped (one
    more per level, depth-first, at most ``max_depth`` flips and ``max_runs``
    reruns) and the first assignment that matches within tolerance is
    adopted.  A flipped-to-kept entry's bias is raised to tau, a
    flipped-to-evicted one's lowered just below it.  The report counts the
    events met and the flips adopted.
    """
    import torch

    w = make_weights(cfg, seed)
    c = make_cache(cfg, w, seed)
    n = cfg.chunk
    per_call = n if not chunked else cfg.n_total
    calls = cfg.n_total // per_call
    layer = device_layer(cfg, w, c, terms=terms, max_tokens=n)
    probe, pc = _probe_layer(cfg, w, c, terms, cfg.n_total)
    od, op = oracle_dims(cfg, terms), oracle_params(w)
    oc = oracle_cache(cfg, c)
    S = cfg.B * cfg.H_kv
    tau = -math.inf if log_p == -math.inf else log_p
    rep = {"y_err": 0.0, "lam_err": 0.0, "borderline": 0, "adopted": 0, "evicted": 0, "calls": calls, "reruns": 0}

    def compact_with(o2, policy, tag, events):
        """Compaction at log_p with the decisions of ``policy``; returns kept lists."""
        for s in range(S):
            lam = o2.lam[s]
            bidx = np.flatnonzero(np.abs(lam - tau) <= BORDER)
            forced = []
            for j in bidx:
                key = (tag, s, int(j))
                own = bool(lam[j] >= tau)
                events.append((key, own))
                forced.append(policy.get(key, own))
            _force(lam, bidx, np.asarray(forced, bool), tau)
        return U.compact(o2, log_p)

    for call in range(calls):
        inp = make_step_inputs(cfg, call, per_call, seed)
        pos0 = probe.cache.next_pos.cpu().numpy().copy()
        plen = probe.cache.seg_len.cpu().numpy().copy()
        probe.prefill(inp.q, inp.k, inp.v, inp.x)
        torch.cuda.synchronize()
        k_gpu = _stored_new(gpu_state(probe), pc.seg_off, plen, cfg, per_call, "K")
        _check_new_keys(cfg, od, inp.k, pos0, k_gpu)
        kept_dev = None
        if chunked:
            y_gpu, _ = layer.prefill_chunked(inp.q, inp.k, inp.v, inp.x, n, log_p)
        else:
            kept_dev = torch.full((layer.cache.total_slots,), -1, dtype=torch.int32, device="cuda")
            y_gpu, _ = layer.prefill_pruned(inp.q, inp.k, inp.v, inp.x, log_p, kept=kept_dev)
        torch.cuda.synchronize()
        y_gpu = y_gpu.float().cpu().numpy()
        g = gpu_state(layer)
        kept_gpu = None if kept_dev is None else kept_dev.cpu().numpy()

        def oracle_call(policy):
            o2 = oc.copy()
            events = []
            y_or = np.zeros((cfg.B, per_call, cfg.H_q, cfg.d))
            if chunked:
                kept_or = None
                for c0 in range(0, per_call, n):
                    c1 = min(per_call, c0 + n)
                    y_or[:, c0:c1] = U.prefill(od, op, o2, inp.q[:, c0:c1], inp.k[:, c0:c1], inp.v[:, c0:c1],
                                               inp.x[:, c0:c1], k_override=k_gpu[:, c0:c1])
                    compact_with(o2, policy, ("c", c0), events)
            else:
                for i in range(per_call):
                    forced = {}

                    def decide(s, lam_new, idx, i=i, forced=forced):
                        live = lam_new >= tau
                        for jj in np.flatnonzero(np.abs(lam_new - tau) <= BORDER):
                            key = ("t", i, s, int(idx[jj]))
                            events.append((key, bool(live[jj])))
                            live[jj] = policy.get(key, bool(live[jj]))
                        forced[s] = (idx, live.copy())
                        return live

                    y_or[:, i], _ = U.decode_step(od, op, o2, inp.q[:, i], inp.k[:, i], inp.v[:, i], inp.x[:, i],
                                                  log_p, decide=decide, k_override=k_gpu[:, i])
                    for s, (idx, live) in forced.items():
                        _force(o2.lam[s], idx, live, tau)
                kept_or = compact_with(o2, policy, ("end",), events)
            y_err = _maxabs(y_gpu, y_or)
            why, lam_err = _cache_mismatch(g, o2, cfg, f"call {call}", kept_gpu, kept_or)
            if why is None and y_err > y_tol(cfg):
                why = f"call {call}: y max-abs error {y_err:.3e}"
            return why, o2, events, y_err, lam_err

        runs = [0]

        def search(policy, depth):
            why, o2, events, y_err, lam_err = oracle_call(policy)
            runs[0] += 1
            if why is None:
                return policy, o2, events, y_err, lam_err, None
            first_why = why
            if depth < max_depth:
                for key, own in events:
                    if key in policy or runs[0] >= max_runs:
                        continue
                    res = search({**policy, key: not own}, depth + 1)
                    if res[5] is None:
                        return res
            return policy, o2, events, y_err, lam_err, first_why

        policy, o2, events, y_err, lam_err, why = search({}, 0)
        rep["reruns"] += runs[0] - 1
        assert why is None, f"{why} ({len(events)} borderline decisions, {runs[0]} oracle runs)"
        rep["borderline"] += len(events)
        rep["adopted"] += len(policy)
        rep["evicted"] += sum(x.size for x in oc.lam) + S * per_call - sum(x.size for x in o2.lam)
        oc = o2
        rep["y_err"] = max(rep["y_err"], y_err)
        rep["lam_err"] = max(rep["lam_err"], lam_err)
    return rep


def run_varlen_parity(cfg: LayerConfig, lens_per_call, terms: int = 7, seed: int = 0) -> dict:
    """ua_prefill_varlen on the GPU against the oracle's per-sequence prefill (R31).

    Call c packs the first lens_per_call[c][b] tokens of sequence b's draw for
    that call.  After every call: y of every packed row (max-abs), rows past
    the packed ones untouched, the stored new keys (one ulp), and the whole
    cache (lengths, rows, biases, key gates, positions, status).
    """
    import torch

    nmax = max(max(l) for l in lens_per_call)
    w = make_weights(cfg, seed)
    c = make_cache(cfg, w, seed)
    layer = device_layer(cfg, w, c, terms=terms, max_tokens=nmax)
    od, op = oracle_dims(cfg, terms), oracle_params(w)
    oc = oracle_cache(cfg, c)
    rep = {"y_err": 0.0, "lam_err": 0.0}
    for call, lens in enumerate(lens_per_call):
        assert len(lens) == cfg.B
        inp = make_step_inputs(cfg, call, nmax, seed)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T = int(cu[-1])
        pack = lambda a: np.concatenate([a[b, : lens[b]] for b in range(cfg.B)], axis=0)
        qp, kp, vp, xp = pack(inp.q), pack(inp.k), pack(inp.v), pack(inp.x)
        len_before = layer.cache.seg_len.cpu().numpy().copy()
        pos0 = layer.cache.next_pos.cpu().numpy().copy()
        y_full = torch.full((T + 8, cfg.H_q, cfg.d), float("nan"), device="cuda")
        layer.prefill_varlen(qp, kp, vp, xp, cu, max_tokens=nmax, y=y_full[:T])
        torch.cuda.synchronize()
        yg = y_full.cpu().numpy()
        assert np.isnan(yg[T:]).all(), f"call {call}: rows past the packed ones were written"
        g = gpu_state(layer)
        k_gpu = np.zeros((T, cfg.H_kv, cfg.d))
        for b in range(cfg.B):
            if lens[b] == 0:
                continue
            rows = np.stack([g["K"][int(c.seg_off[b * cfg.H_kv + h]) + int(len_before[b * cfg.H_kv + h]):][: lens[b]]
                             for h in range(cfg.H_kv)], axis=1)
            _check_new_keys(cfg, od, kp[None, cu[b]:cu[b + 1]], pos0[b:b + 1], rows[None])
            k_gpu[cu[b]:cu[b + 1]] = rows
        y_or = U.prefill_varlen(od, op, oc, qp, kp, vp, xp, cu, k_override=k_gpu)
        y_err = _maxabs(yg[:T], y_or)
        lam_err = _compare_cache(layer, oc, cfg, f"call {call}")
        rep["y_err"] = max(rep["y_err"], y_err)
        rep["lam_err"] = max(rep["lam_err"], lam_err)
        assert y_err <= y_tol(cfg), f"call {call}: y max-abs error {y_err:.3e}"
        assert lam_err <= 1e-4, f"call {call}: log-bias error {lam_err:.3e}"
    return rep
