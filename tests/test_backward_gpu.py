"""Backward of the decay-mask and attention part (ua_attention_backward) against the oracle.

The oracle is fp64 autograd through the forward of one training chunk from an
empty cache (paperlayer.ai summary, sections 4.2 and Appendix C: a decay-mask
kernel paired with a fused attention kernel for training).  The device takes
the same bf16-rounded (or fp32) inputs and works in fp32 throughout, so the
comparison is of fp32 arithmetic against fp64 on identical numbers.  Each
gradient is compared element by element, scaled by its largest oracle value:
max |g - g_ref| <= TOL * max |g_ref|.  TOL is 2e-4: the longest fp32 chains
are sums of N <= 256 products after an exp, each step with a relative error
of a few 2^-24 (the exp and log intrinsics are within 2 ulp), so the scaled
error stays below (N + d) * 2^-22 ~ 1e-4 for these sizes.

Inputs (ua_inputs.make_grad_inputs): rotated queries q~ ~ N(0, 1); stored
keys k~ unit vectors (the keys are L2-normalised before RoPE, which keeps the
norm); v, dO ~ N(0, 1); log-gates log sigmoid(z) with z ~ N(b_h, 32) (hidden
2048 and gate weights of variance 1/64) and a per-head bias b_h uniform in
[-4, 0], as in the 1B-shape chunked prefill.
"""

import math

import numpy as np
import pytest

import oracle as U

pytestmark = pytest.mark.gpu

TOL = 2e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_pruning_amd import load

    load()


def _inputs(B, N, Hq, Hkv, d, bf16, seed, dup_pairs=0):
    from ua_inputs import make_grad_inputs

    return make_grad_inputs(B, N, Hq, Hkv, d, bf16, seed, repeat_pairs=dup_pairs).astuple()


def _device_backward(q, k, v, lq, lk, lb, dO, terms, bf16, scale=0.0):
    import torch

    import kv_cache_pruning_amd as K

    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    dt = torch.bfloat16 if bf16 else torch.float32
    dims = K.make_dims(B, Hq, Hkv, d, 2048, bf16=bf16, terms=terms, sm_scale=scale)
    dev = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", t)
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    lqd, lkd, lbd, dOd = dev(lq), dev(lk), dev(lb), dev(dO)
    outs = [torch.full(a.shape, float("nan"), device="cuda") for a in (q, k, v, lq, lk, lb)]
    nb = K.ua_backward_workspace_bytes(dims, N)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    K.ua_attention_backward(dims, N, qd, kd, vd, lqd, lkd, lbd, dOd, *outs, ws, nb)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def _oracle_backward(q, k, v, lq, lk, lb, dO, terms, scale):
    refs = [np.zeros(a.shape) for a in (q, k, v, lq, lk, lb)]
    for b in range(q.shape[0]):
        g = U.ua_grad.attention_backward(q[b].astype(np.float64), k[b].astype(np.float64), v[b].astype(np.float64),
                                         lq[b].astype(np.float64), lk[b].astype(np.float64),
                                         lb[b].astype(np.float64), dO[b].astype(np.float64), terms, scale)
        for r, x in zip(refs, g):
            r[b] = x
    return refs


NAMES = ("dq", "dk", "dv", "dlq", "dlk", "dlb")


def _check(B, N, Hq, Hkv, d, bf16, terms, seed, dup_pairs=0, scale=0.0):
    print(f"[backward] B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} bf16={bf16} terms={terms} seed={seed}", flush=True)
    ins = _inputs(B, N, Hq, Hkv, d, bf16, seed, dup_pairs)
    got = _device_backward(*ins, terms, bf16, scale)
    ref = _oracle_backward(*ins, terms, scale if scale > 0 else 1.0 / math.sqrt(d))
    errs = {}
    for name, g, r in zip(NAMES, got, ref):
        assert np.isfinite(g).all(), name
        m = np.abs(r).max()
        errs[name] = float(np.abs(g - r).max() / m) if m > 0 else float(np.abs(g).max())
    print("  scaled errors", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
    for name, e in errs.items():
        assert e <= TOL, (name, e)
    return got, ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("G", [1, 4])
def test_backward_all_terms(d, bf16, G):
    _check(2, 150, 2 * G, 2, d, bf16, U.TERMS_ALL, seed=10 + d + G)


@pytest.mark.parametrize("terms", [0, U.TERM_Q, U.TERM_K, U.TERM_SIM, U.TERM_Q | U.TERM_K, U.TERM_K | U.TERM_SIM])
def test_backward_term_subsets(terms):
    got, _ = _check(1, 97, 4, 2, 64, True, terms, seed=40 + terms)
    # a gate the enabled terms do not use gets exactly zero
    for name, bit in (("dlq", U.TERM_Q), ("dlk", U.TERM_K), ("dlb", U.TERM_SIM)):
        if not terms & bit:
            assert not got[NAMES.index(name)].any(), name


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 128, 129, 256])
def test_backward_lengths(N):
    _check(1, N, 8, 1, 64, True, U.TERMS_ALL, seed=70 + N)


def test_backward_group_of_eight_and_custom_scale():
    _check(1, 120, 16, 2, 128, True, U.TERMS_ALL, seed=5, scale=0.07)


def test_backward_repeated_keys_clamp():
    """Keys repeated at a norm above 1 reach the similarity clamp (min(s^2, 1) = 1)."""
    k = _inputs(2, 90, 4, 2, 64, True, 6, dup_pairs=12)[1].astype(np.float64)
    s = np.einsum("bthd,bjhd->bhtj", k, k)
    assert (np.tril(s * s, -1) >= 1.0).sum() >= 10  # distinct pairs at the clamp
    _check(2, 90, 4, 2, 64, True, U.TERMS_ALL, seed=6, dup_pairs=12)


def test_backward_single_token():
    """One token: its softmax is over itself, so dq = dk = 0 (dS = dO.v - dO.o, zero up to fp32
    rounding of two equal dot products), dv = dO summed over the group, and the gates get 0."""
    q, k, v, lq, lk, lb, dO = _inputs(1, 1, 4, 1, 64, False, 9)
    got = _device_backward(q, k, v, lq, lk, lb, dO, U.TERMS_ALL, False)
    assert np.abs(got[0]).max() <= 1e-5 and np.abs(got[1]).max() <= 1e-5
    np.testing.assert_allclose(got[2][0, 0, 0], dO[0, 0].sum(axis=0), rtol=1e-6, atol=1e-6)
    assert not got[3].any() and not got[4].any() and not got[5].any()


def test_backward_1b_chunk():
    """The 1B-shape training chunk (32 / 8 heads, d 64, N 1024): one sequence against the oracle in full."""
    B, N, Hq, Hkv, d = 1, 1024, 32, 8, 64
    _check(B, N, Hq, Hkv, d, True, U.TERMS_ALL, seed=123)


def test_backward_bench_size_sampled():
    """The bench's workload (B = 2, N = 4096, 32 / 8 heads, d = 64, bf16): the device backward of the
    whole batch, and one (sequence, KV head) group of it against the oracle in full."""
    import torch

    import kv_cache_pruning_amd as K

    B, N, Hq, Hkv, d = 2, 4096, 32, 8, 64
    G = Hq // Hkv
    print(f"[backward] bench size B={B} N={N} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    q, k, v, lq, lk, lb, dO = _inputs(B, N, Hq, Hkv, d, True, 0)
    got = _device_backward(q, k, v, lq, lk, lb, dO, U.TERMS_ALL, True)
    b, h = 1, 5
    qs, hs = slice(h * G, (h + 1) * G), slice(h, h + 1)
    ref = U.ua_grad.attention_backward(q[b, :, qs].astype(np.float64), k[b, :, hs].astype(np.float64),
                                       v[b, :, hs].astype(np.float64), lq[b, :, hs].astype(np.float64),
                                       lk[b, :, hs].astype(np.float64), lb[b, :, hs].astype(np.float64),
                                       dO[b, :, qs].astype(np.float64), U.TERMS_ALL, 1.0 / math.sqrt(d))
    parts = (got[0][b, :, qs], got[1][b, :, hs], got[2][b, :, hs], got[3][b, :, hs], got[4][b, :, hs],
             got[5][b, :, hs])
    for name, g, r in zip(NAMES, parts, ref):
        assert np.isfinite(g).all(), name
        e = float(np.abs(g - r).max() / np.abs(r).max())
        print(f"  {name} scaled error {e:.2e}", flush=True)
        assert e <= TOL, (name, e)
    for a in got:  # every other group is finite too
        assert np.isfinite(a).all()
