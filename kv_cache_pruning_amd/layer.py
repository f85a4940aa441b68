"""Device-side containers for one UA layer: weights, cache and workspace.

Plain torch tensors on the GPU plus the ctypes structs that point at them.
Every call goes straight to libua.so; nothing here computes.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib as L


def _dev(a, dtype, device) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a)).to(device=device, dtype=dtype).contiguous()


@dataclass
class LayerShape:
    B: int
    H_q: int
    H_kv: int
    d: int
    D: int
    r: int = 16
    bf16: bool = True
    y_bf16: bool = False
    terms: int = L.UA_TERMS_ALL
    rope_base: float = 10000.0
    sm_scale: float = 0.0

    def dims(self) -> L.ua_dims:
        return L.make_dims(self.B, self.H_q, self.H_kv, self.d, self.D, self.r, self.bf16, self.y_bf16, self.terms,
                           self.rope_base, self.sm_scale)

    @property
    def dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.bf16 else torch.float32


class DeviceWeights:
    def __init__(self, shape: LayerShape, W_dec, b_dec, W_dn, W_up, b_up=None, device="cuda"):
        dt = shape.dtype
        self.W_dec = _dev(W_dec, dt, device)
        self.b_dec = _dev(b_dec, torch.float32, device)
        self.W_dn = _dev(W_dn, dt, device)
        self.W_up = _dev(W_up, dt, device)
        self.b_up = None if b_up is None else _dev(b_up, torch.float32, device)
        self.params = L.make_params(self.W_dec, self.b_dec, self.W_dn, self.W_up, self.b_up)


class DeviceCache:
    """Slot-layout cache: K/V [slots, d], logbias/kgate [slots], segment table."""

    def __init__(self, shape: LayerShape, K, V, logbias, kgate, seg_off, seg_len, seg_cap, next_pos, device="cuda"):
        dt = shape.dtype
        self.shape = shape
        self.K = _dev(K, dt, device)
        self.V = _dev(V, dt, device)
        self.logbias = _dev(logbias, torch.float32, device)
        self.kgate = _dev(kgate, torch.float32, device)
        self.seg_off = _dev(seg_off, torch.int64, device)
        self.seg_len = _dev(seg_len, torch.int32, device)
        self.seg_cap = _dev(seg_cap, torch.int32, device)
        self.next_pos = _dev(next_pos, torch.int32, device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.max_seg_cap = int(np.max(seg_cap))
        self.struct = L.make_cache(self.K, self.V, self.logbias, self.kgate, self.seg_off, self.seg_len, self.seg_cap,
                                   self.next_pos, self.status)

    @property
    def total_slots(self) -> int:
        return int(self.K.shape[0])


class Workspace:
    def __init__(self, shape: LayerShape, cache: DeviceCache, max_tokens: int = 1, device="cuda"):
        n = L.ua_workspace_bytes(shape.dims(), max_tokens, cache.total_slots, cache.max_seg_cap)
        if n == 0:
            raise L.UAError("ua_workspace_bytes rejected the layer shape")
        self.nbytes = n
        self.buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
        self.ptr = (self.buf.data_ptr() + 255) // 256 * 256  # 256-byte aligned start
        L.ua_workspace_init(self.ptr, n)  # counters must start at zero


class Layer:
    """One UA layer bound to a cache: decode / prefill / compact through the C ABI."""

    def __init__(self, shape: LayerShape, weights: DeviceWeights, cache: DeviceCache, max_tokens: int = 1,
                 device="cuda", workspace: Optional[Workspace] = None):
        self.shape = shape
        self.dims = shape.dims()
        self.w = weights
        self.cache = cache
        self.ws = workspace if workspace is not None else Workspace(shape, cache, max_tokens, device)
        self.device = device

    def _tokens(self, q, k, v, x):
        dt = self.shape.dtype
        ts = [t if (isinstance(t, torch.Tensor) and t.device.type == "cuda" and t.dtype == dt and t.is_contiguous())
              else _dev(t, dt, self.device) for t in (q, k, v, x)]
        return ts, L.make_tokens(*ts)

    def decode_step(self, q, k, v, x, log_p: float, y: Optional[torch.Tensor] = None, stream=None):
        s = self.shape
        ts, tok = self._tokens(q, k, v, x)
        if y is None:
            y = torch.empty((s.B, s.H_q, s.d), dtype=torch.bfloat16 if s.y_bf16 else torch.float32,
                            device=self.device)
        L.ua_decode_step(self.dims, self.w.params, self.cache.struct, tok, log_p, y, self.ws.ptr, self.ws.nbytes,
                         stream)
        return y, ts

    def decode_compact_step(self, q, k, v, x, log_p: float, y: Optional[torch.Tensor] = None,
                            kept: Optional[torch.Tensor] = None, stream=None):
        """One decode step and the compaction of every segment in one launch."""
        s = self.shape
        ts, tok = self._tokens(q, k, v, x)
        if y is None:
            y = torch.empty((s.B, s.H_q, s.d), dtype=torch.bfloat16 if s.y_bf16 else torch.float32,
                            device=self.device)
        L.ua_decode_compact_step(self.dims, self.w.params, self.cache.struct, tok, log_p, y, kept, self.ws.ptr,
                                 self.ws.nbytes, stream)
        return y, ts

    def decode_compact_step_noalloc(self, q, k, v, x, log_p: float, y: torch.Tensor,
                                    kept: Optional[torch.Tensor] = None, stream=None):
        """decode_compact_step on the library's own per-GPU workspace: the call
        allocates nothing, so y (and kept, if wanted) must be given."""
        ts, tok = self._tokens(q, k, v, x)
        L.ua_decode_compact_step_noalloc(self.dims, self.w.params, self.cache.struct, tok, log_p, y, kept, stream)
        return y, ts

    def prefill(self, q, k, v, x, y: Optional[torch.Tensor] = None, stream=None):
        s = self.shape
        n = q.shape[1]
        ts, tok = self._tokens(q, k, v, x)
        if y is None:
            y = torch.empty((s.B, n, s.H_q, s.d), dtype=torch.bfloat16 if s.y_bf16 else torch.float32,
                            device=self.device)
        L.ua_prefill(self.dims, self.w.params, self.cache.struct, tok, n, y, self.ws.ptr, self.ws.nbytes, stream)
        return y, ts

    def qk_norm(self, q, k, w_q=None, w_k=None, eps: float = 1e-6, stream=None):
        """Qwen3-style RMS normalisation of q [B, n, H_q, d] and k [B, n, H_kv, d] in place
        (device copies in the layer's dtype are made first if needed); returns (q, k)."""
        dt = self.shape.dtype
        q = q if (isinstance(q, torch.Tensor) and q.device.type == "cuda" and q.dtype == dt and q.is_contiguous()) \
            else _dev(q, dt, self.device)
        k = k if (isinstance(k, torch.Tensor) and k.device.type == "cuda" and k.dtype == dt and k.is_contiguous()) \
            else _dev(k, dt, self.device)
        wq = None if w_q is None else _dev(w_q, torch.float32, self.device)
        wk = None if w_k is None else _dev(w_k, torch.float32, self.device)
        L.ua_qk_norm(self.dims, wq, wk, eps, q, k, q.shape[1], stream)
        return q, k

    def prefill_pruned(self, q, k, v, x, log_p: float, y: Optional[torch.Tensor] = None,
                       kept: Optional[torch.Tensor] = None, stream=None):
        """Prefill that leaves entries below log_p out of the softmax, then compacts."""
        s = self.shape
        n = q.shape[1]
        ts, tok = self._tokens(q, k, v, x)
        if y is None:
            y = torch.empty((s.B, n, s.H_q, s.d), dtype=torch.bfloat16 if s.y_bf16 else torch.float32,
                            device=self.device)
        L.ua_prefill_pruned(self.dims, self.w.params, self.cache.struct, tok, n, log_p, y, kept, self.ws.ptr,
                            self.ws.nbytes, stream)
        return y, ts

    def prefill_chunked(self, q, k, v, x, chunk: int, log_p: float, y: Optional[torch.Tensor] = None, stream=None):
        """Dense prefill in chunks of `chunk` tokens, compacting at log_p after each."""
        s = self.shape
        n = q.shape[1]
        ts, tok = self._tokens(q, k, v, x)
        if y is None:
            y = torch.empty((s.B, n, s.H_q, s.d), dtype=torch.bfloat16 if s.y_bf16 else torch.float32,
                            device=self.device)
        L.ua_prefill_chunked(self.dims, self.w.params, self.cache.struct, tok, n, chunk, log_p, y, self.ws.ptr,
                             self.ws.nbytes, stream)
        return y, ts

    def prefill_varlen(self, q, k, v, x, cu_seqlens, max_tokens: Optional[int] = None,
                       y: Optional[torch.Tensor] = None, stream=None):
        """Prefill of a packed batch: sequence b appends rows cu_seqlens[b] .. cu_seqlens[b + 1] of q [T, H_q, d],
        k, v [T, H_kv, d] and x [T, D]; y is [T, H_q, d].  max_tokens defaults to the longest sequence."""
        s = self.shape
        T = q.shape[0]
        cu_host = [int(c) for c in (cu_seqlens.tolist() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens)]
        if max_tokens is None:
            max_tokens = max(b - a for a, b in zip(cu_host[:-1], cu_host[1:]))
        cu = torch.tensor(cu_host, dtype=torch.int32, device=self.device)
        ts, tok = self._tokens(q, k, v, x)
        if y is None:
            y = torch.empty((T, s.H_q, s.d), dtype=torch.bfloat16 if s.y_bf16 else torch.float32, device=self.device)
        L.ua_prefill_varlen(self.dims, self.w.params, self.cache.struct, tok, cu, T, max_tokens, y, self.ws.ptr,
                            self.ws.nbytes, stream)
        return y, ts

    def compact(self, log_p: float, kept: Optional[torch.Tensor] = None, stream=None):
        L.ua_compact(self.dims, self.cache.struct, log_p, kept, self.ws.ptr, self.ws.nbytes, stream)
        return kept


def layer_from_arrays(B: int, H_q: int, H_kv: int, d: int, D: int, r: int, bf16: bool, weights, cache,
                      terms: int = L.UA_TERMS_ALL, max_tokens: int = 1, y_bf16: bool = False,
                      workspace: Optional[Workspace] = None, device="cuda") -> Layer:
    """A Layer from host arrays.

    ``weights`` holds W_dec, b_dec, W_dn, W_up, b_up; ``cache`` holds K, V,
    lam (log-biases), lk (key gates), seg_off, seg_len, seg_cap, next_pos
    (attributes of plain objects, e.g. dataclasses).  Copies go to the device.
    """
    shape = LayerShape(B=B, H_q=H_q, H_kv=H_kv, d=d, D=D, r=r, bf16=bf16, y_bf16=y_bf16, terms=terms)
    w, c = weights, cache
    dw = DeviceWeights(shape, w.W_dec, w.b_dec, w.W_dn, w.W_up, w.b_up, device=device)
    dc = DeviceCache(shape, c.K, c.V, c.lam, c.lk, c.seg_off, c.seg_len, c.seg_cap, c.next_pos, device=device)
    return Layer(shape, dw, dc, max_tokens=max_tokens, device=device, workspace=workspace)
