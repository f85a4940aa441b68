"""Shared parity machinery: the same seeded inputs go to the oracle and to the
HIP path (through the C ABI), and outputs are compared with the tolerances
of the spec: y max-abs 1e-2 (bf16) / 1e-4 (fp32); log-biases
|d| <= 1e-4 * max(|oracle|, 1); keep masks identical except entries within
1e-4 of log p, where the oracle adopts the GPU's value; compaction exact.
"""

from __future__ import annotations

import math
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
    from kv_cache_pruning_amd.layer import DeviceCache, DeviceWeights, Layer, LayerShape

    shape = LayerShape(B=cfg.B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, D=cfg.D, r=cfg.r, bf16=cfg.bf16, y_bf16=y_bf16,
                       terms=terms)
    dw = DeviceWeights(shape, w.W_dec, w.b_dec, w.W_dn, w.W_up, w.b_up)
    dc = DeviceCache(shape, c.K, c.V, c.lam, c.lk, c.seg_off, c.seg_len, c.seg_cap, c.next_pos)
    return Layer(shape, dw, dc, max_tokens=max_tokens)


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
    def borderline(self):
        return sum(r.n_border for r in self.reports)


def gpu_state(layer):
    """Copy the device cache back to numpy (fp64 values)."""
    c = layer.cache
    return dict(
        K=c.K.float().cpu().numpy().astype(np.float64),
        V=c.V.float().cpu().numpy().astype(np.float64),
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
            live_g = lam_g >= tau
            border = np.abs(lam_new - tau) <= BORDER
            border_log[s] = (idx[border], lam_g[border])
            mismatch = (live_o != live_g) & ~border
            assert not mismatch.any(), f"step {step} seg {s}: keep mask differs away from the threshold"
            return np.where(border, live_g, live_o)

        y_or, info = U.decode_step(od, op, oc, q, k, v, x, log_p, decide=decide, k_override=k_use)
        # adopt borderline GPU values so both trajectories continue from the same state
        nb = 0
        for s, (bidx, lamg) in border_log.items():
            oc.lam[s][bidx] = lamg
            nb += len(bidx)
        y_err = float(np.max(np.abs(y_gpu - y_or)))
        lam_err = 0.0
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
                lam_err = max(lam_err, float(np.max(np.abs(lg[fin] - lo[fin]) / np.maximum(np.abs(lo[fin]), 1.0))))
            n_upd += idx.size
            n_dead += int((~it["live"]).sum())
        # lengths, positions, status
        assert np.array_equal(g["seg_len"], oc.lengths()), f"step {step}: segment lengths differ"
        assert np.array_equal(g["next_pos"], oc.next_pos), f"step {step}: positions differ"
        assert g["status"] == oc.status, f"step {step}: status differs"
        run.reports.append(StepReport(step, y_err, lam_err, nb, n_upd, n_dead))
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
