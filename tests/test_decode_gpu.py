"""Decode-step and compaction parity: HIP path (C ABI) vs the fp64 oracle.

Every step compares y, the updated log-biases, the keep masks (borderline
entries within 1e-4 of log p adopted from the GPU and counted), segment
lengths, positions and status; every compaction compares the kept-index list
exactly and the moved rows bit for bit.
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


def _run(cfg, steps, p, **kw):
    from tests.harness import run_decode_parity

    print(f"[decode parity] {cfg.name} B={cfg.B} steps={steps} p={p} {kw}", flush=True)
    run = run_decode_parity(cfg, steps, math.log(p) if p > 0 else -math.inf, **kw)
    print(f"  max |dy| {run.max_y_err:.2e}  max rel dLambda {run.max_lam_err:.2e} (floor 1e-6: "
          f"{run.max_lam_err_strict:.2e})  borderline {run.borderline}  dead {sum(r.n_dead for r in run.reports)}", flush=True)
    return run


def test_tiny_decode_fp32_all_steps():
    """Tiny fp32 layer, 256 steps from an empty cache, compaction every step."""
    cfg = config("tiny-decode-f32")
    run = _run(cfg, cfg.steps, cfg.p)
    assert sum(r.n_dead for r in run.reports) > 0


def test_1b_decode_full_batch():
    cfg = config("1b-decode")
    _run(cfg, 12, cfg.p)


def test_1b_decode_small_many_steps():
    cfg = config("1b-decode", B=2)
    _run(cfg, 40, cfg.p)


def test_3b_decode_full_batch():
    cfg = config("3b-decode")
    _run(cfg, 6, cfg.p)


def test_ragged_decode_full_batch():
    cfg = config("ragged-decode")
    _run(cfg, 4, cfg.p)


def test_ragged_decode_small_many_steps():
    cfg = config("ragged-decode", B=4)
    _run(cfg, 24, cfg.p)


@pytest.mark.parametrize("terms", [0, 1, 2, 4, 3, 5, 6])
def test_term_subsets(terms):
    cfg = config("1b-decode", B=2)
    _run(cfg, 4, cfg.p, terms=terms)


def test_lazy_compaction_and_p0():
    cfg = config("1b-decode", B=2)
    _run(cfg, 10, cfg.p, compact_every=4)
    _run(cfg, 6, 0.0, compact_every=0)


@pytest.mark.parametrize("G,d", [(1, 64), (2, 128), (8, 64), (4, 128), (3, 64), (8, 128)])
def test_group_and_head_dims(G, d):
    cfg = config("1b-decode", B=2, H_kv=2, H_q=2 * G, d=d, D=256, len_mean=200.0, len_max=600)
    _run(cfg, 6, cfg.p)


def test_fp32_cache_128():
    cfg = config("tiny-decode-f32", B=3, H_q=6, H_kv=2, d=128, D=128, steps=40)
    _run(cfg, 40, 0.15)


def test_segment_full_sets_status():
    """Capacity reached: status bit 0 set, append skipped, output still formed."""
    cfg = config("tiny-decode-f32", B=2, H_q=2, H_kv=1, steps=8)
    from tests import harness as H
    import ua_inputs as G

    orig = G.make_cache

    def small(cfg_, w_, seed=0, extra=None):
        c = orig(cfg_, w_, seed, extra=5)
        return c

    H.make_cache = small
    try:
        run = _run(cfg, 20, 0.0, compact_every=0)
    finally:
        H.make_cache = orig
    assert len(run.reports) == 20


def test_shared_workspace_across_cache_sizes():
    """Two layers of one shape whose caches differ in size share one workspace.

    The calls interleave (decode + compaction on A, then on B) and must give
    exactly what each layer gives with a workspace of its own.
    """
    import torch

    from kv_cache_pruning_amd.layer import DeviceCache, DeviceWeights, Layer, LayerShape, Workspace
    from tests.harness import gpu_state
    from ua_inputs import make_cache, make_step_inputs, make_weights

    cfg = config("1b-decode", B=2)
    shape = LayerShape(B=cfg.B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, D=cfg.D, r=cfg.r, bf16=True)
    w = make_weights(cfg, 0)
    dw = DeviceWeights(shape, w.W_dec, w.b_dec, w.W_dn, w.W_up, w.b_up)
    inits = [make_cache(cfg, w, seed=0, extra=16), make_cache(cfg, w, seed=1, extra=4096)]
    assert inits[0].slots != inits[1].slots

    def dev(ci):
        return DeviceCache(shape, ci.K, ci.V, ci.lam, ci.lk, ci.seg_off, ci.seg_len, ci.seg_cap, ci.next_pos)

    shared_caches = [dev(ci) for ci in inits]
    ws = Workspace(shape, max(shared_caches, key=lambda c: c.total_slots), 1)
    shared = [Layer(shape, dw, c, workspace=ws) for c in shared_caches]
    private = [Layer(shape, dw, dev(ci)) for ci in inits]
    log_p = math.log(cfg.p)
    for step in range(6):
        inp = make_step_inputs(cfg, step, 1, 0)
        args = (inp.q[:, 0], inp.k[:, 0], inp.v[:, 0], inp.x[:, 0])
        ys, yp = [], []
        for L in shared:
            ys.append(L.decode_step(*args, log_p)[0])
            L.compact(log_p)
        for L in private:
            yp.append(L.decode_step(*args, log_p)[0])
            L.compact(log_p)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(ys[i], yp[i]), f"step {step} layer {i}: y differs with a shared workspace"
            gs, gp = gpu_state(shared[i]), gpu_state(private[i])
            assert np.array_equal(gs["seg_len"], gp["seg_len"]) and gs["status"] == gp["status"] == 0
            for o, n in zip(gs["seg_off"], gs["seg_len"]):
                assert np.array_equal(gs["lam"][o : o + n], gp["lam"][o : o + n])
                assert np.array_equal(gs["K"][o : o + n], gp["K"][o : o + n])


# ---- decode step and compaction in one launch (ua_decode_compact_step) ----
def _run_fused(cfg, steps, p, **kw):
    from tests.harness import run_fused_parity

    print(f"[fused parity] {cfg.name} B={cfg.B} steps={steps} p={p} {kw}", flush=True)
    run = run_fused_parity(cfg, steps, math.log(p) if p > 0 else -math.inf, **kw)
    print(f"  max |dy| {run.max_y_err:.2e}  max rel dLambda {run.max_lam_err:.2e} (floor 1e-6: "
          f"{run.max_lam_err_strict:.2e})  borderline {run.borderline}  evicted {sum(r.n_dead for r in run.reports)}", flush=True)
    return run


def test_fused_tiny_fp32_all_steps():
    cfg = config("tiny-decode-f32")
    run = _run_fused(cfg, cfg.steps, cfg.p)
    assert sum(r.n_dead for r in run.reports) > 0


def test_fused_1b_decode_full_batch():
    _run_fused(config("1b-decode"), 12, 0.15)


def test_fused_3b_decode_full_batch():
    _run_fused(config("3b-decode"), 6, 0.15)


def test_fused_ragged_decode():
    _run_fused(config("ragged-decode", B=8), 4, 0.05)


def test_fused_p0_keeps_everything():
    _run_fused(config("1b-decode", B=2), 6, 0.0)


@pytest.mark.parametrize("terms", [0, 1, 2, 4, 6])
def test_fused_term_subsets(terms):
    _run_fused(config("1b-decode", B=2), 4, 0.15, terms=terms)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (24, 8), (64, 8)])
def test_fused_group_sizes(hq, hkv):
    _run_fused(config("1b-decode", B=2, H_q=hq, H_kv=hkv), 4, 0.15)


def test_fused_group8_head128():
    """Group size 8 at head dim 128 (64 query heads over 8 KV heads, 3B-shape cache)."""
    _run_fused(config("3b-decode", B=2, H_q=64, H_kv=8), 6, 0.15)


def test_group8_head128_3b_cache():
    _run(config("3b-decode", B=2, H_q=64, H_kv=8), 6, 0.15)


# ---- every configuration over its stated number of steps (eviction is monotone:
# an entry once evicted never returns, so long runs are what exercise it) ----
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["1b-decode", "3b-decode", "ragged-decode"])
def test_all_steps_two_calls(name):
    """ua_decode_step then ua_compact, every step of the configuration at its full batch."""
    cfg = config(name)
    run = _run(cfg, cfg.steps, cfg.p)
    assert len(run.reports) == cfg.steps
    assert sum(r.n_dead for r in run.reports) > 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["1b-decode", "3b-decode", "ragged-decode"])
def test_all_steps_fused(name):
    """ua_decode_compact_step, every step of the configuration at its full batch."""
    cfg = config(name)
    run = _run_fused(cfg, cfg.steps, cfg.p)
    assert len(run.reports) == cfg.steps
    assert sum(r.n_dead for r in run.reports) > 0


@pytest.mark.parametrize("p", [0.0, 0.02])
def test_fused_equals_two_calls_when_segments_fill(p):
    """Segments with room for three more entries: once full, the fused call
    sets status bit 0 and skips the append exactly as decode_step followed by
    ua_compact does (same outputs, rows, biases, kept lists, status)."""
    import torch

    from tests.harness import device_layer, gpu_state
    from ua_inputs import make_cache, make_step_inputs, make_weights

    cfg = config("1b-decode", B=2)
    w = make_weights(cfg, 0)
    c = make_cache(cfg, w, 0, extra=3)
    fused, two = device_layer(cfg, w, c), device_layer(cfg, w, c)
    log_p = math.log(p) if p > 0 else -math.inf
    slots = fused.cache.total_slots
    kf = torch.full((slots,), -1, dtype=torch.int32, device="cuda")
    kt = torch.full((slots,), -1, dtype=torch.int32, device="cuda")
    for step in range(8):
        inp = make_step_inputs(cfg, step, 1, 0)
        args = (inp.q[:, 0], inp.k[:, 0], inp.v[:, 0], inp.x[:, 0])
        kf.fill_(-1)
        kt.fill_(-1)
        print(f"[fused vs two calls] p={p} step {step}", flush=True)
        yf, _ = fused.decode_compact_step(*args, log_p, kept=kf)
        yt, _ = two.decode_step(*args, log_p)
        two.compact(log_p, kept=kt)
        torch.cuda.synchronize()
        assert torch.equal(yf, yt), f"step {step}: y differs"
        gf, gt = gpu_state(fused), gpu_state(two)
        assert gf["status"] == gt["status"], f"step {step}: status {gf['status']} vs {gt['status']}"
        assert np.array_equal(gf["seg_len"], gt["seg_len"]) and np.array_equal(gf["next_pos"], gt["next_pos"])
        kfn, ktn = kf.cpu().numpy(), kt.cpu().numpy()
        for o, n in zip(gf["seg_off"], gf["seg_len"]):
            for name in ("K", "V", "lam", "lk"):
                assert np.array_equal(gf[name][o : o + n], gt[name][o : o + n]), f"step {step}: {name} differs"
            if p > 0:
                assert np.array_equal(kfn[o : o + n], ktn[o : o + n]), f"step {step}: kept lists differ"
    assert gf["status"] & 1, "no segment reached its capacity"
