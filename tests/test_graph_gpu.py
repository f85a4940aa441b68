"""Decode + compaction captured in a HIP graph replays exactly like eager calls.

The library launches kernels only (no memset nodes), keeps lengths on the
device and resets its workspace counters itself, so a captured step can be
replayed.  Each replay is compared with an eager run on a copy of the same
cache, with eager work and synchronisations between replays.
"""

import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["decode+compact", "decode_compact_step"])
def test_graph_replay_matches_eager(fused):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.harness import device_layer
    from ua_inputs import config, make_cache, make_step_inputs, make_weights

    cfg = config("1b-decode", B=4)
    w = make_weights(cfg, 0)
    c = make_cache(cfg, w, 0)
    eager = device_layer(cfg, w, c)
    graphed = device_layer(cfg, w, c)
    log_p = math.log(cfg.p)
    dt = torch.bfloat16
    static = [torch.empty(0)] * 4
    inp0 = make_step_inputs(cfg, 0, 1, 0)
    static = [torch.from_numpy(np.ascontiguousarray(a[:, 0])).to("cuda", dt) for a in (inp0.q, inp0.k, inp0.v, inp0.x)]
    y_g = torch.empty((cfg.B, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        if fused:
            graphed.decode_compact_step(*static, log_p, y=y_g)
        else:
            graphed.decode_step(*static, log_p, y=y_g)
            graphed.compact(log_p)
    torch.cuda.synchronize()
    for step in range(8):
        inp = make_step_inputs(cfg, step, 1, 0)
        host = [np.ascontiguousarray(a[:, 0]) for a in (inp.q, inp.k, inp.v, inp.x)]
        for dst, src in zip(static, host):
            dst.copy_(torch.from_numpy(src).to(dt))
        g.replay()
        if fused:
            y_e, _ = eager.decode_compact_step(*host, log_p)
        else:
            y_e, _ = eager.decode_step(*host, log_p)
            eager.compact(log_p)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {step}: y differs"
        for name in ("seg_len", "next_pos", "status"):
            assert torch.equal(getattr(graphed.cache, name), getattr(eager.cache, name)), f"replay {step}: {name}"
        n = eager.cache.seg_len.cpu().numpy()
        off = eager.cache.seg_off.cpu().numpy()
        lg, le = graphed.cache.logbias.cpu().numpy(), eager.cache.logbias.cpu().numpy()
        Kg, Ke = graphed.cache.K.cpu(), eager.cache.K.cpu()
        Vg, Ve = graphed.cache.V.cpu(), eager.cache.V.cpu()
        for o, m in zip(off, n):
            assert np.array_equal(lg[o : o + m], le[o : o + m]), f"replay {step}: log-biases differ"
            assert torch.equal(Kg[o : o + m], Ke[o : o + m]), f"replay {step}: keys differ"
            assert torch.equal(Vg[o : o + m], Ve[o : o + m]), f"replay {step}: values differ"
        _ = torch.ones(1000, device="cuda").sum().item()  # unrelated eager work between replays
