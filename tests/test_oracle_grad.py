"""Pins of the fp64 gradient reference (oracle/ua_grad.py).

- Its forward equals the pinned numpy oracle's dense forms (O5 column sums,
  O7 attention) for every subset of decay terms.
- Its autograd gradients equal central finite differences of that forward.
- With no decay term the gradients of q~, k~, v are those of torch's own fp64
  causal scaled-dot-product attention, and the gate gradients vanish.
"""

import math

import numpy as np
import pytest
import torch

import oracle as U
from oracle import ua_grad as UG


def _case(N=10, Hq=4, Hkv=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    qt = rng.normal(0, 1, (N, Hq, d))
    kt = rng.normal(0, 1, (N, Hkv, d))
    kt /= np.linalg.norm(kt, axis=-1, keepdims=True)
    v = rng.normal(0, 1, (N, Hkv, d))
    lq, lk, lb = (rng.uniform(-3.0, -0.05, (N, Hkv)) for _ in range(3))
    dO = rng.normal(0, 1, (N, Hq, d))
    return qt, kt, v, lq, lk, lb, dO


@pytest.mark.parametrize("terms", [0, 1, 2, 4, 3, 5, 6, 7])
def test_forward_equals_dense_oracle(terms):
    qt, kt, v, lq, lk, lb, _ = _case(seed=terms)
    N, Hq, d = qt.shape
    Hkv = kt.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    o = UG.attention_forward(*(torch.tensor(x) for x in (qt, kt, v, lq, lk, lb)), terms, scale).numpy()
    rows = np.arange(N)
    for h in range(Hkv):
        lam = U.dense_logbias(terms, kt[:, h], lq[:, h], lk[:, h], lb[:, h], rows)
        ref = U.dense_attention(qt[:, h * G:(h + 1) * G], kt[:, h], v[:, h], lam, rows, scale)
        assert np.allclose(o[:, h * G:(h + 1) * G], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("terms", [7, 5, 2])
def test_gradients_equal_finite_differences(terms):
    qt, kt, v, lq, lk, lb, dO = _case(N=5, Hq=2, Hkv=1, d=4, seed=11 + terms)
    scale = 0.5
    grads = UG.attention_backward(qt, kt, v, lq, lk, lb, dO, terms, scale)
    base = [qt, kt, v, lq, lk, lb]

    def f(xs):
        o = UG.attention_forward(*(torch.tensor(x) for x in xs), terms, scale).numpy()
        return float(np.sum(o * dO))

    h = 1e-6
    for which, g in enumerate(grads):
        x = base[which]
        for idx in np.ndindex(x.shape):
            xp = [b.copy() for b in base]
            xm = [b.copy() for b in base]
            xp[which][idx] += h
            xm[which][idx] -= h
            fd = (f(xp) - f(xm)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, g[idx])


def test_no_decay_matches_torch_sdpa_gradients():
    qt, kt, v, lq, lk, lb, dO = _case(N=9, Hq=4, Hkv=2, d=8, seed=3)
    scale = 0.3
    dq, dk, dv, dlq, dlk, dlb = UG.attention_backward(qt, kt, v, lq, lk, lb, dO, 0, scale)
    assert not dlq.any() and not dlk.any() and not dlb.any()
    Q = torch.tensor(qt).permute(1, 0, 2)[None].requires_grad_()
    K0 = torch.tensor(kt).requires_grad_()
    V0 = torch.tensor(v).requires_grad_()
    K = K0.permute(1, 0, 2).repeat_interleave(2, dim=0)[None]
    V = V0.permute(1, 0, 2).repeat_interleave(2, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    (o[0].permute(1, 0, 2) * torch.tensor(dO)).sum().backward()
    assert np.allclose(dq, Q.grad[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, K0.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, V0.grad.numpy(), rtol=1e-10, atol=1e-12)
