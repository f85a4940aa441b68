"""Chunked-prefill parity: HIP path (C ABI) vs the fp64 oracle.

Small cases compare every output, every cached log-bias, the stored keys,
values and key gates after each call against the oracle's token-by-token
prefill.  The full 1B prefill workload (B=2, 32/8 heads, 16 calls of 1024
tokens) is checked on sampled rows and on the final log-bias vectors of
sampled segments, computed one by one from the oracle's dense definitions.
Cross-path identities: chunked == one-shot prefill, and decode at p = 0
reproduces prefill.
"""

import math

import numpy as np
import pytest

from ua_inputs import config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_pruning_amd import load

    load()  # fails loudly if libua.so is missing


def _run(cfg, **kw):
    from tests.harness import run_prefill_parity

    print(f"[prefill parity] {cfg.name} B={cfg.B} H={cfg.H_q}/{cfg.H_kv} d={cfg.d} chunk={cfg.chunk} "
          f"n_total={cfg.n_total} {kw}", flush=True)
    rep = run_prefill_parity(cfg, **kw)
    print(f"  max |dy| {rep['y_err']:.2e}  max rel dLambda {rep['lam_err']:.2e}  max dlk {rep['lk_err']:.2e}",
          flush=True)
    return rep


SMALL = dict(B=1, H_q=8, H_kv=2, D=256, n_total=256, chunk=128)


def test_prefill_small_two_calls():
    _run(config("1b-prefill", **SMALL))


def test_prefill_ragged_chunks():
    """Calls of 100 tokens: partial token blocks, lengths off the 64-key grid."""
    _run(config("1b-prefill", B=2, H_q=8, H_kv=2, D=256, n_total=300, chunk=100))


def test_prefill_per_xcd_ticket_queues():
    """8 and 16 segments: workgroups take tickets from one queue per XCD."""
    _run(config("1b-prefill", B=4, H_q=8, H_kv=2, D=256, n_total=300, chunk=150))
    _run(config("1b-prefill", B=2, H_q=16, H_kv=8, D=256, n_total=200, chunk=100, len_kind="lognormal",
                len_mean=120.0, len_min=16, len_max=400, nominal=400, lam_p0=0.15))
    # the lock-step kernel: head dim 128 (group 3), and group 8 at head dim 64
    _run(config("1b-prefill", B=1, H_q=24, H_kv=8, d=128, D=256, n_total=160, chunk=80))
    _run(config("1b-prefill", B=1, H_q=64, H_kv=8, D=256, n_total=160, chunk=80))


def test_prefill_single_token_calls():
    _run(config("1b-prefill", B=1, H_q=4, H_kv=1, D=64, n_total=5, chunk=1))


def test_prefill_on_populated_cache():
    """Cached entries carry stored biases that the call's column sums extend."""
    cfg = config("1b-prefill", B=2, H_q=8, H_kv=2, D=256, n_total=192, chunk=96, len_kind="lognormal",
                 len_mean=120.0, len_min=16, len_max=400, nominal=400, lam_p0=0.15)
    _run(cfg)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (6, 2), (16, 2)])
def test_prefill_group_sizes_d64(hq, hkv):
    _run(config("1b-prefill", B=1, H_q=hq, H_kv=hkv, D=128, n_total=160, chunk=80))


@pytest.mark.parametrize("hq,hkv", [(2, 2), (6, 2), (8, 2)])
def test_prefill_head_dim_128(hq, hkv):
    _run(config("1b-prefill", B=1, H_q=hq, H_kv=hkv, d=128, D=256, n_total=160, chunk=80))


@pytest.mark.parametrize("terms", [0, 1, 2, 4, 3, 5, 6])
def test_prefill_term_subsets(terms):
    _run(config("1b-prefill", **SMALL), terms=terms)


def test_prefill_bf16_output():
    _run(config("1b-prefill", **SMALL), y_bf16=True)


@pytest.mark.parametrize("q_scale", [4.0, 8.0])
def test_prefill_large_query_norms(q_scale):
    """Queries of norm ~32 and ~64: waves whose scaled norms leave the fixed
    softmax reference's range run the running-maximum path (some waves at 4,
    all at 8)."""
    _run(config("1b-prefill", q_scale=q_scale, **SMALL))


def test_prefill_1b_heads_full_batch():
    _run(config("1b-prefill", n_total=384, chunk=192))


def test_prefill_segment_without_room():
    """A segment lacking room for the call: status bit, zero outputs, segment untouched."""
    import torch

    from tests.harness import device_layer, gpu_state
    from ua_inputs import make_cache, make_step_inputs, make_weights

    cfg = config("1b-prefill", B=2, H_q=4, H_kv=2, D=64, n_total=64, chunk=64)
    w = make_weights(cfg)
    c = make_cache(cfg, w)
    c.seg_cap[1] = 48  # segment 1 (b=0, h=1) cannot take 64 tokens
    layer = device_layer(cfg, w, c, max_tokens=cfg.chunk)
    inp = make_step_inputs(cfg, 0, cfg.chunk)
    y, _ = layer.prefill(inp.q, inp.k, inp.v, inp.x)
    torch.cuda.synchronize()
    g = gpu_state(layer)
    assert g["status"] & 1
    assert list(g["seg_len"]) == [64, 0, 64, 64]
    assert list(g["next_pos"]) == [64, 64]
    yy = y.cpu().numpy()
    G = cfg.H_q // cfg.H_kv
    assert np.all(yy[0, :, G:2 * G] == 0.0)
    assert np.all(np.isfinite(yy)) and np.any(yy[0, :, :G] != 0.0)


def test_chunked_equals_one_shot():
    """Four calls of 128 tokens == one call of 512 (both on the GPU)."""
    import torch

    from tests.harness import device_layer, gpu_state
    from ua_inputs import make_cache, make_step_inputs, make_weights

    cfg = config("1b-prefill", B=2, H_q=8, H_kv=2, D=256, n_total=512, chunk=128)
    w = make_weights(cfg)
    c = make_cache(cfg, w)
    whole = make_step_inputs(cfg, 0, 512)
    one = device_layer(cfg, w, c, max_tokens=512)
    y1, _ = one.prefill(whole.q, whole.k, whole.v, whole.x)
    many = device_layer(cfg, w, c, max_tokens=128)
    ys = []
    for i in range(4):
        sl = slice(128 * i, 128 * (i + 1))
        yi, _ = many.prefill(whole.q[:, sl], whole.k[:, sl], whole.v[:, sl], whole.x[:, sl])
        ys.append(yi)
    torch.cuda.synchronize()
    y4 = torch.cat(ys, dim=1)
    err = float((y1 - y4).abs().max())
    g1, g4 = gpu_state(one), gpu_state(many)
    assert np.array_equal(g1["seg_len"], g4["seg_len"])
    l1, l4 = g1["lam"], g4["lam"]
    lam_err = float(np.max(np.abs(l1 - l4) / np.maximum(np.abs(l1), 1.0)))
    print(f"chunked vs one-shot: max |dy| {err:.2e}, max rel dLambda {lam_err:.2e}")
    assert err <= 1e-2 and lam_err <= 1e-4


def test_decode_at_p0_reproduces_prefill():
    """Token-by-token decode with p = 0 gives the prefill's outputs and biases."""
    import torch

    from tests.harness import device_layer, gpu_state
    from ua_inputs import make_cache, make_step_inputs, make_weights

    cfg = config("1b-prefill", B=2, H_q=8, H_kv=2, D=256, n_total=160, chunk=160)
    w = make_weights(cfg)
    c = make_cache(cfg, w)
    inp = make_step_inputs(cfg, 0, 160)
    pre = device_layer(cfg, w, c, max_tokens=160)
    yp, _ = pre.prefill(inp.q, inp.k, inp.v, inp.x)
    dec = device_layer(cfg, w, c)
    yd = []
    for t in range(160):
        yt, _ = dec.decode_step(inp.q[:, t], inp.k[:, t], inp.v[:, t], inp.x[:, t], -math.inf)
        yd.append(yt.clone())
    torch.cuda.synchronize()
    yd = torch.stack(yd, dim=1)
    err = float((yp - yd).abs().max())
    gp, gd = gpu_state(pre), gpu_state(dec)
    assert np.array_equal(gp["seg_len"], gd["seg_len"]) and np.array_equal(gp["next_pos"], gd["next_pos"])
    assert np.array_equal(gp["K"], gd["K"]) or np.max(np.abs(gp["K"] - gd["K"])) <= 2.0**-8
    lam_err = float(np.max(np.abs(gp["lam"] - gd["lam"]) / np.maximum(np.abs(gd["lam"]), 1.0)))
    print(f"decode(p=0) vs prefill: max |dy| {err:.2e}, max rel dLambda {lam_err:.2e}")
    assert err <= 1e-2 and lam_err <= 1e-4


@pytest.mark.timeout(900)
def test_prefill_1b_full_workload_with_eviction():
    """The full 1B prefill workload (16 calls of 1024 tokens, 2 x 8 segments):
    every segment's final log-biases, 16 sampled rows of every call, then the
    eviction at p = 0.05 (kept lists exact given the mask, the mask equal to
    the oracle's away from log p)."""
    from tests.harness import run_prefill_full

    cfg = config("1b-prefill")
    rep = run_prefill_full(cfg, rows_per_call=16, log_p=math.log(cfg.p))
    print(f"full 1b-prefill: max |dy| {rep['y_err']:.2e} over {rep['n_rows']} rows in {rep['segments']} segments, "
          f"max rel dLambda(final) {rep['lam_err']:.2e}; eviction at p={cfg.p}: {rep['kept']} kept, "
          f"{rep['borderline']} borderline", flush=True)
    assert rep["segments"] == cfg.B * cfg.H_kv


# ---------------------------------------------------------------------------
# pruned prefill (threshold mask + compaction) and chunk-boundary eviction
# ---------------------------------------------------------------------------
POPULATED = dict(len_kind="lognormal", len_mean=120.0, len_min=16, len_max=400, nominal=400, lam_p0=0.15)


def _run_pruned(cfg, log_p, chunked=False, seeds=(0, 1), **kw):
    """Fixed seeds; keep decisions within 1e-4 of log p are searched for the
    GPU's choice (the harness reruns the oracle with them flipped) and counted."""
    from tests.harness import run_pruned_prefill_parity

    for seed in seeds:
        print(f"[pruned prefill] chunked={chunked} {cfg.name} B={cfg.B} H={cfg.H_q}/{cfg.H_kv} d={cfg.d} "
              f"chunk={cfg.chunk} n_total={cfg.n_total} log_p={log_p:.4f} seed={seed}", flush=True)
        rep = run_pruned_prefill_parity(cfg, log_p, chunked=chunked, seed=seed, **kw)
        print(f"  max |dy| {rep['y_err']:.2e}  max rel dLambda {rep['lam_err']:.2e}  evicted {rep['evicted']}  "
              f"borderline {rep['borderline']}  adopted {rep['adopted']}  reruns {rep['reruns']}", flush=True)
        assert rep["evicted"] > 0, "the case evicts nothing"


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 64), (16, 2, 64), (4, 2, 128)])
def test_pruned_prefill_equals_decode(hq, hkv, d):
    """ua_prefill_pruned == token-by-token decode at p, then compaction (both attention kernels)."""
    cfg = config("1b-prefill", B=2, H_q=hq, H_kv=hkv, d=d, D=256, n_total=192, chunk=64, **POPULATED)
    _run_pruned(cfg, math.log(0.15))


def test_pruned_prefill_ragged_call_from_empty_cache():
    cfg = config("1b-prefill", B=2, H_q=8, H_kv=2, D=256, n_total=200, chunk=100)
    _run_pruned(cfg, math.log(0.3))


def test_pruned_prefill_term_subset():
    cfg = config("1b-prefill", B=1, H_q=8, H_kv=2, D=256, n_total=128, chunk=128, **POPULATED)
    _run_pruned(cfg, math.log(0.15), terms=3)


@pytest.mark.parametrize("n_total,chunk", [(256, 128), (200, 64)])
def test_chunk_boundary_eviction(n_total, chunk):
    """ua_prefill_chunked == per chunk: dense prefill, then compaction at p."""
    cfg = config("1b-prefill", B=2, H_q=8, H_kv=2, D=256, n_total=n_total, chunk=chunk, **POPULATED)
    _run_pruned(cfg, math.log(0.05), chunked=True)
