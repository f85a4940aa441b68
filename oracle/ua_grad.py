"""fp64 gradient reference for the decay-mask and attention part of a UA layer.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

The forward here is O4-O7 of ``ua_ref`` (paperlayer.ai summary, sections 4,
4.1 and 4.2; ai4snews page, Figure 1 caption) for one sequence of a training
chunk that starts from an empty cache, written with plain torch fp64 CPU ops so
that torch.autograd gives the gradients of the paper's training kernels (its
Appendix C pairs a decay-mask kernel with an attention kernel).  Inputs are
the rotated queries q~ [N, H_q, d], the stored keys k~ [N, H_kv, d], the
values v [N, H_kv, d] and the log-gates lq, lk, lb [N, H_kv]; the output is
the attention output o [N, H_q, d] before the output gate.  The tests pin this
forward to ``ua_ref`` and its gradients to central finite differences.

Reading (R29): u = min(s^2, 1) passes the gradient where s^2 < 1 and none
where the clamp holds (s^2 >= 1 only for equal keys).
"""

from __future__ import annotations

import torch

from .ua_ref import TERM_K, TERM_Q, TERM_SIM


def _log1mexp(lam: torch.Tensor) -> torch.Tensor:
    """log(1 - e^lam) for lam <= 0, differentiable (R16's two branches)."""
    near = lam > -0.6931471805599453
    a = torch.log(-torch.expm1(torch.where(near, lam, torch.full_like(lam, -1.0))))
    b = torch.log1p(-torch.exp(torch.where(near, torch.full_like(lam, -1.0), lam)))
    return torch.where(near, a, b)


def attention_forward(qt, kt, v, lq, lk, lb, terms: int, scale: float) -> torch.Tensor:
    """O4-O7 for one sequence from an empty cache: o [N, H_q, d] (fp64 torch)."""
    N, Hq, d = qt.shape
    Hkv = kt.shape[1]
    G = Hq // Hkv
    n_terms = bin(terms & 7).count("1")
    causal = torch.tril(torch.ones(N, N, dtype=torch.bool))
    strict = torch.tril(torch.ones(N, N, dtype=torch.bool), diagonal=-1)
    outs = []
    for h in range(Hkv):
        K = kt[:, h]
        if n_terms:
            lam = torch.zeros(N, N, dtype=qt.dtype)
            if terms & TERM_Q:
                lam = lam + lq[:, h][:, None]
            if terms & TERM_K:
                lam = lam + lk[:, h][None, :]
            if terms & TERM_SIM:
                s = K @ K.T
                s2 = s * s
                u = torch.where(s2 < 1.0, s2, torch.ones_like(s2))
                lam = lam + lb[:, h][:, None] + torch.log(torch.where(strict, u, torch.ones_like(u)))
            lam = lam / n_terms
            A = torch.where(strict, _log1mexp(torch.where(strict, lam, torch.full_like(lam, -1.0))),
                            torch.zeros_like(lam))
        else:
            A = torch.zeros(N, N, dtype=qt.dtype)
        Lam = torch.cumsum(A, dim=0)  # Lam[i, j] = sum_{t <= i} A[t, j], A[t, j] = 0 for t <= j
        for a in range(G):
            e = scale * (qt[:, h * G + a] @ K.T) + Lam
            e = torch.where(causal, e, torch.full_like(e, float("-inf")))
            P = torch.softmax(e, dim=1)
            outs.append(P @ v[:, h])
    return torch.stack(outs, dim=1)


def attention_backward(qt, kt, v, lq, lk, lb, dO, terms: int, scale: float):
    """Gradients (dq~, dk~, dv, dlq, dlk, dlb) of <dO, o> by fp64 autograd (numpy in, numpy out)."""
    args = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (qt, kt, v, lq, lk, lb)]
    o = attention_forward(*args, terms, scale)
    (o * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    # an input the enabled terms do not use gets a zero gradient
    return tuple(a.grad.numpy() if a.grad is not None else torch.zeros_like(a).detach().numpy() for a in args)
