"""ua_decode_compact_step_noalloc (the library's own per-GPU workspace) gives
exactly what ua_decode_compact_step gives with a caller workspace.

Two calls in a row share the GPU's array, the second on a smaller layer and
cache; then a third repeats the first shape to show nothing from the
smaller call lingers.  A cache whose step would need more than the array
holds is rejected before anything is launched.
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


def _pair(cfg, seed, extra):
    """Two layers on identical copies of one cache: one for each entry point."""
    from kv_cache_pruning_amd.layer import DeviceCache, DeviceWeights, Layer, LayerShape
    from ua_inputs import make_cache, make_weights

    shape = LayerShape(B=cfg.B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, D=cfg.D, r=cfg.r, bf16=cfg.bf16)
    w = make_weights(cfg, seed)
    dw = DeviceWeights(shape, w.W_dec, w.b_dec, w.W_dn, w.W_up, w.b_up)
    ci = make_cache(cfg, w, seed=seed, extra=extra)

    def layer():
        c = DeviceCache(shape, ci.K, ci.V, ci.lam, ci.lk, ci.seg_off, ci.seg_len, ci.seg_cap, ci.next_pos)
        return Layer(shape, dw, c)

    return shape, layer(), layer()


def _step(cfg, shape, ref, nal, step):
    import torch

    from kv_cache_pruning_amd import _lib as L
    from tests.harness import gpu_state
    from ua_inputs import make_step_inputs

    inp = make_step_inputs(cfg, step, 1, 0)
    args = (inp.q[:, 0], inp.k[:, 0], inp.v[:, 0], inp.x[:, 0])
    log_p = math.log(cfg.p)
    n = ref.cache.total_slots
    kr = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    kn = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    ydt = torch.bfloat16 if shape.y_bf16 else torch.float32
    yr = torch.empty((shape.B, shape.H_q, shape.d), dtype=ydt, device="cuda")
    yn = torch.full_like(yr, float("nan"))
    ref.decode_compact_step(*args, log_p, y=yr, kept=kr)
    nal.decode_compact_step_noalloc(*args, log_p, yn, kn)
    torch.cuda.synchronize()
    assert torch.equal(yr, yn), f"{cfg.name} step {step}: y differs"
    gr, gn = gpu_state(ref), gpu_state(nal)
    assert gr["status"] == gn["status"] == 0
    assert np.array_equal(gr["seg_len"], gn["seg_len"]) and np.array_equal(gr["next_pos"], gn["next_pos"])
    kr, kn = kr.cpu().numpy(), kn.cpu().numpy()
    for o, m in zip(gr["seg_off"], gr["seg_len"]):
        assert np.array_equal(kr[o : o + m], kn[o : o + m]), f"{cfg.name} step {step}: kept lists differ"
        for f in ("lam", "lk", "K", "V"):
            assert np.array_equal(gr[f][o : o + m], gn[f][o : o + m]), f"{cfg.name} step {step}: {f} differs"
    return int(gr["seg_len"].sum())


def test_noalloc_matches_workspace_entry_point_two_sizes():
    big = config("3b-decode", B=8)
    small = config("1b-decode", B=2)
    pb = _pair(big, 0, 64)
    ps = _pair(small, 1, 16)
    assert pb[1].cache.total_slots > ps[1].cache.total_slots
    print(f"[noalloc] {big.name} B={big.B} slots={pb[1].cache.total_slots}, then {small.name} B={small.B} "
          f"slots={ps[1].cache.total_slots}", flush=True)
    n1 = _step(big, *pb, 0)
    n2 = _step(small, *ps, 0)
    n3 = _step(big, *pb, 1)
    print(f"  live after the calls: {n1}, {n2}, {n3}", flush=True)


def test_noalloc_rejects_a_step_beyond_the_array():
    import torch

    from kv_cache_pruning_amd import _lib as L
    from kv_cache_pruning_amd.layer import DeviceCache, DeviceWeights, Layer, LayerShape
    from ua_inputs import make_weights

    cfg = config("ragged-decode")
    shape = LayerShape(B=cfg.B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, D=cfg.D, r=cfg.r, bf16=True)
    S, cap = cfg.B * cfg.H_kv, 8192  # 4.2M slots: the step needs more than the array
    need = L.ua_workspace_bytes(shape.dims(), 1, S * cap, cap)
    assert need > L.UA_NOALLOC_SCRATCH_BYTES
    seg_off = np.arange(S, dtype=np.int64) * cap
    seg_len = np.full(S, 100, np.int32)
    z = np.zeros((S * cap,), np.float32)
    Kz = np.zeros((S * cap, cfg.d), np.float32)
    w = make_weights(cfg, 0)
    dw = DeviceWeights(shape, w.W_dec, w.b_dec, w.W_dn, w.W_up, w.b_up)
    c = DeviceCache(shape, Kz, Kz, z, z, seg_off, seg_len, np.full(S, cap, np.int32), np.full(cfg.B, 100, np.int32))
    layer = Layer(shape, dw, c)
    q = torch.zeros((cfg.B, cfg.H_q, cfg.d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((cfg.B, cfg.H_kv, cfg.d), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((cfg.B, cfg.D), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((cfg.B, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(L.UAError, match="workspace"):
        layer.decode_compact_step_noalloc(q, kv, kv, x, math.log(cfg.p), y)
    torch.cuda.synchronize()
    assert int(c.status.item()) == 0 and np.array_equal(c.seg_len.cpu().numpy(), seg_len)
