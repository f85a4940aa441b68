"""Qwen3-style normalised queries and keys (ua_qk_norm) against the oracle.

The kernel's output is compared with the oracle's fp64 RMS normalisation
rounded to the token dtype (bf16: within one ulp, as the fp32 sum of squares
may round a tie the other way; fp32: 2e-6 relative).  End to end, a prefill
on normalised inputs is compared with the oracle's prefill on the same
normalisation of the raw inputs.
"""

import math

import numpy as np
import pytest

import oracle as U
from ua_inputs import config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_pruning_amd import load

    load()


def _layer(cfg, n):
    from tests.harness import device_layer
    from ua_inputs import make_cache, make_weights

    w = make_weights(cfg, 0)
    c = make_cache(cfg, w, 0)
    return device_layer(cfg, w, c, max_tokens=n), w, c


@pytest.mark.parametrize("d,bf16", [(64, True), (128, True), (64, False), (128, False)])
def test_qk_norm_matches_oracle(d, bf16):
    import torch

    from tests.harness import ulp_bf16

    cfg = config("1b-prefill", B=2, H_q=8, H_kv=2, d=d, D=256, n_total=37, chunk=37, bf16=bf16)
    print(f"[qk_norm] d={d} bf16={bf16}", flush=True)
    layer, _, _ = _layer(cfg, 37)
    rng = np.random.default_rng(3)
    q = rng.normal(0, 2.0, (cfg.B, 37, cfg.H_q, d)).astype(np.float32)
    k = rng.normal(0, 0.5, (cfg.B, 37, cfg.H_kv, d)).astype(np.float32)
    wq = rng.normal(1, 0.3, d).astype(np.float32)
    wk = rng.normal(1, 0.3, d).astype(np.float32)
    dt = torch.bfloat16 if bf16 else torch.float32
    qd = torch.from_numpy(q).to("cuda", dt)
    kd = torch.from_numpy(k).to("cuda", dt)
    qin = qd.double().cpu().numpy()
    kin = kd.double().cpu().numpy()
    layer.qk_norm(qd, kd, wq, wk, 1e-6)
    torch.cuda.synchronize()
    for got, x, w in ((qd, qin, wq), (kd, kin, wk)):
        ref = U.qk_rmsnorm(x, w.astype(np.float64), 1e-6)
        g = got.double().cpu().numpy()
        if bf16:
            ref_r = U.bf16_round(ref)
            assert np.all(np.abs(g - ref_r) <= ulp_bf16(ref_r) * 1.0001), "more than one bf16 ulp off"
        else:
            assert np.max(np.abs(g - ref) / np.maximum(np.abs(ref), 1e-3)) <= 2e-6


def test_qk_norm_null_weight_leaves_tensor():
    import torch

    cfg = config("1b-prefill", B=1, H_q=4, H_kv=2, D=256, n_total=8, chunk=8)
    layer, _, _ = _layer(cfg, 8)
    q = torch.randn(1, 8, 4, 64, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 8, 2, 64, device="cuda").to(torch.bfloat16)
    q0, k0 = q.clone(), k.clone()
    layer.qk_norm(q, k, None, np.ones(64, np.float32))
    torch.cuda.synchronize()
    assert torch.equal(q, q0) and not torch.equal(k, k0)


def test_prefill_with_normalised_queries_and_keys():
    """ua_qk_norm then ua_prefill == oracle prefill on qk_rmsnorm'd inputs (rounded to bf16)."""
    import torch

    from tests.harness import oracle_cache, oracle_dims, oracle_params, y_tol, _maxabs, gpu_state, _stored_new
    from ua_inputs import make_step_inputs

    cfg = config("1b-prefill", B=2, H_q=8, H_kv=2, D=256, n_total=96, chunk=96)
    layer, w, c = _layer(cfg, 96)
    rng = np.random.default_rng(5)
    wq = rng.normal(1, 0.3, cfg.d).astype(np.float32)
    wk = rng.normal(1, 0.3, cfg.d).astype(np.float32)
    inp = make_step_inputs(cfg, 0, 96, 0)
    qd = torch.from_numpy(inp.q).to("cuda", torch.bfloat16)
    kd = torch.from_numpy(inp.k).to("cuda", torch.bfloat16)
    layer.qk_norm(qd, kd, wq, wk, 1e-6)
    len0 = layer.cache.seg_len.cpu().numpy().copy()
    y, _ = layer.prefill(qd, kd, inp.v, inp.x)
    torch.cuda.synchronize()
    # the oracle normalises the same raw inputs itself; it takes the GPU-normalised
    # bits only where the two roundings of a value may differ (checked above)
    qn = U.bf16_round(U.qk_rmsnorm(inp.q, wq.astype(np.float64)))
    kn = U.bf16_round(U.qk_rmsnorm(inp.k, wk.astype(np.float64)))
    qg = qd.double().cpu().numpy()
    kg = kd.double().cpu().numpy()
    from tests.harness import ulp_bf16
    assert np.all(np.abs(qg - qn) <= ulp_bf16(qn) * 1.0001) and np.all(np.abs(kg - kn) <= ulp_bf16(kn) * 1.0001)
    od, op, oc = oracle_dims(cfg), oracle_params(w), oracle_cache(cfg, c)
    k_st = _stored_new(gpu_state(layer), c.seg_off, len0, cfg, 96, "K")
    y_or = U.prefill(od, op, oc, qg, kg, inp.v, inp.x, k_override=k_st)
    err = _maxabs(y.float().cpu().numpy(), y_or)
    print(f"  prefill on normalised q/k: max |dy| {err:.2e}", flush=True)
    assert err <= y_tol(cfg)
