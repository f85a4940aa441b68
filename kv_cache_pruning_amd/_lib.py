"""ctypes binding of libua.so: the C-ABI entry points under the same names.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Buffers are torch CUDA tensors (device memory and streams); their
data pointers are passed straight through.  If the library is missing the
import of any entry point raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("UA_LIB", os.path.join(HERE, "libua.so"))

UA_OK, UA_ERR_INVALID_ARG, UA_ERR_UNSUPPORTED, UA_ERR_WORKSPACE, UA_ERR_HIP = range(5)
UA_F32, UA_BF16 = 0, 1
UA_TERM_Q, UA_TERM_K, UA_TERM_SIM, UA_TERMS_ALL = 1, 2, 4, 7
UA_STATUS_SEGMENT_FULL, UA_STATUS_WAIT_TIMEOUT, UA_STATUS_BAD_LENGTH = 1, 2, 4
UA_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = (
    "ua_workspace_bytes",
    "ua_workspace_init",
    "ua_decode_step",
    "ua_decode_compact_step",
    "ua_decode_compact_step_noalloc",
    "ua_prefill",
    "ua_prefill_pruned",
    "ua_prefill_chunked",
    "ua_prefill_varlen",
    "ua_qk_norm",
    "ua_backward_workspace_bytes",
    "ua_attention_backward",
    "ua_compact",
    "ua_status_string",
    "ua_abi_version",
)


class ua_dims(C.Structure):
    _fields_ = [
        ("B", C.c_int32),
        ("H_q", C.c_int32),
        ("H_kv", C.c_int32),
        ("d_head", C.c_int32),
        ("d_model", C.c_int32),
        ("gate_rank", C.c_int32),
        ("dtype", C.c_int32),
        ("y_dtype", C.c_int32),
        ("terms", C.c_int32),
        ("reserved0", C.c_int32),
        ("rope_base", C.c_double),
        ("sm_scale", C.c_float),
        ("reserved1", C.c_float),
    ]


class ua_params(C.Structure):
    _fields_ = [("W_dec", C.c_void_p), ("b_dec", C.c_void_p), ("W_dn", C.c_void_p), ("W_up", C.c_void_p),
                ("b_up", C.c_void_p)]


class ua_tokens(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("x", C.c_void_p)]


class ua_grad_inputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("q", "k", "v", "lq", "lk", "lb", "dO")]


class ua_grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("dq", "dk", "dv", "dlq", "dlk", "dlb")]


class ua_cache(C.Structure):
    _fields_ = [
        ("K", C.c_void_p),
        ("V", C.c_void_p),
        ("logbias", C.c_void_p),
        ("kgate", C.c_void_p),
        ("seg_off", C.c_void_p),
        ("seg_len", C.c_void_p),
        ("seg_cap", C.c_void_p),
        ("next_pos", C.c_void_p),
        ("status", C.c_void_p),
        ("total_slots", C.c_int64),
    ]


class UAError(RuntimeError):
    pass


_lib = None


def load(path: Optional[str] = None) -> C.CDLL:
    """Load libua.so (once) and declare the entry points' signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise UAError(f"libua.so not found at {p}; build it with `python -m kv_cache_pruning_amd.build`")
    lib = C.CDLL(p)
    P = C.POINTER
    lib.ua_workspace_bytes.argtypes = [P(ua_dims), C.c_int32, C.c_int64, C.c_int32]
    lib.ua_workspace_bytes.restype = C.c_size_t
    lib.ua_workspace_init.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p]
    lib.ua_workspace_init.restype = C.c_int
    lib.ua_decode_step.argtypes = [P(ua_dims), P(ua_params), P(ua_cache), P(ua_tokens), C.c_float, C.c_void_p,
                                   C.c_void_p, C.c_size_t, C.c_void_p]
    lib.ua_decode_step.restype = C.c_int
    lib.ua_decode_compact_step.argtypes = [P(ua_dims), P(ua_params), P(ua_cache), P(ua_tokens), C.c_float,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.ua_decode_compact_step.restype = C.c_int
    lib.ua_decode_compact_step_noalloc.argtypes = [P(ua_dims), P(ua_params), P(ua_cache), P(ua_tokens), C.c_float,
                                                   C.c_void_p, C.c_void_p, C.c_void_p]
    lib.ua_decode_compact_step_noalloc.restype = C.c_int
    lib.ua_prefill.argtypes = [P(ua_dims), P(ua_params), P(ua_cache), P(ua_tokens), C.c_int32, C.c_void_p,
                               C.c_void_p, C.c_size_t, C.c_void_p]
    lib.ua_prefill.restype = C.c_int
    lib.ua_prefill_pruned.argtypes = [P(ua_dims), P(ua_params), P(ua_cache), P(ua_tokens), C.c_int32, C.c_float,
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.ua_prefill_pruned.restype = C.c_int
    lib.ua_prefill_chunked.argtypes = [P(ua_dims), P(ua_params), P(ua_cache), P(ua_tokens), C.c_int32, C.c_int32,
                                       C.c_float, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.ua_prefill_chunked.restype = C.c_int
    lib.ua_prefill_varlen.argtypes = [P(ua_dims), P(ua_params), P(ua_cache), P(ua_tokens), C.c_void_p, C.c_int32,
                                      C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.ua_prefill_varlen.restype = C.c_int
    lib.ua_qk_norm.argtypes = [P(ua_dims), C.c_void_p, C.c_void_p, C.c_float, C.c_void_p, C.c_void_p, C.c_int32,
                               C.c_void_p]
    lib.ua_qk_norm.restype = C.c_int
    lib.ua_backward_workspace_bytes.argtypes = [P(ua_dims), C.c_int32]
    lib.ua_backward_workspace_bytes.restype = C.c_size_t
    lib.ua_attention_backward.argtypes = [P(ua_dims), C.c_int32, P(ua_grad_inputs), P(ua_grads), C.c_void_p,
                                          C.c_size_t, C.c_void_p]
    lib.ua_attention_backward.restype = C.c_int
    lib.ua_compact.argtypes = [P(ua_dims), P(ua_cache), C.c_float, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.ua_compact.restype = C.c_int
    lib.ua_status_string.argtypes = [C.c_int32]
    lib.ua_status_string.restype = C.c_char_p
    lib.ua_abi_version.argtypes = []
    lib.ua_abi_version.restype = C.c_int32
    if path is None:
        _lib = lib
    return lib


def _check(code: int, what: str) -> None:
    if code != UA_OK:
        raise UAError(f"{what}: {load().ua_status_string(code).decode()} ({code})")


# ---------------------------------------------------------------------------
# the entry points, same names as the C ABI
# ---------------------------------------------------------------------------
def ua_workspace_bytes(dims: ua_dims, max_tokens_per_call: int, total_slots: int, max_seg_cap: int) -> int:
    return int(load().ua_workspace_bytes(C.byref(dims), max_tokens_per_call, total_slots, max_seg_cap))


def ua_workspace_init(ws, ws_bytes: int, stream=None) -> None:
    _check(load().ua_workspace_init(_ptr(ws), ws_bytes, _stream(stream)), "ua_workspace_init")


def ua_decode_step(dims, params, cache, tokens, log_p: float, y, ws, ws_bytes: int, stream=None) -> None:
    _check(load().ua_decode_step(C.byref(dims), C.byref(params), C.byref(cache), C.byref(tokens), float(log_p),
                                 _ptr(y), _ptr(ws), ws_bytes, _stream(stream)), "ua_decode_step")


def ua_decode_compact_step(dims, params, cache, tokens, log_p: float, y, kept_idx, ws, ws_bytes: int,
                           stream=None) -> None:
    _check(load().ua_decode_compact_step(C.byref(dims), C.byref(params), C.byref(cache), C.byref(tokens),
                                         float(log_p), _ptr(y), _ptr(kept_idx), _ptr(ws), ws_bytes,
                                         _stream(stream)), "ua_decode_compact_step")


def ua_decode_compact_step_noalloc(dims, params, cache, tokens, log_p: float, y, kept_idx, stream=None) -> None:
    _check(load().ua_decode_compact_step_noalloc(C.byref(dims), C.byref(params), C.byref(cache), C.byref(tokens),
                                                 float(log_p), _ptr(y), _ptr(kept_idx), _stream(stream)),
           "ua_decode_compact_step_noalloc")


def ua_prefill(dims, params, cache, tokens, n_tokens: int, y, ws, ws_bytes: int, stream=None) -> None:
    _check(load().ua_prefill(C.byref(dims), C.byref(params), C.byref(cache), C.byref(tokens), int(n_tokens),
                             _ptr(y), _ptr(ws), ws_bytes, _stream(stream)), "ua_prefill")


def ua_prefill_pruned(dims, params, cache, tokens, n_tokens: int, log_p: float, y, kept_idx, ws, ws_bytes: int,
                      stream=None) -> None:
    _check(load().ua_prefill_pruned(C.byref(dims), C.byref(params), C.byref(cache), C.byref(tokens), int(n_tokens),
                                    float(log_p), _ptr(y), _ptr(kept_idx), _ptr(ws), ws_bytes, _stream(stream)),
           "ua_prefill_pruned")


def ua_prefill_varlen(dims, params, cache, tokens, cu_seqlens, total_tokens: int, max_tokens: int, y, ws,
                      ws_bytes: int, stream=None) -> None:
    _check(load().ua_prefill_varlen(C.byref(dims), C.byref(params), C.byref(cache), C.byref(tokens), _ptr(cu_seqlens),
                                    int(total_tokens), int(max_tokens), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "ua_prefill_varlen")


def ua_prefill_chunked(dims, params, cache, tokens, n_tokens: int, chunk: int, log_p: float, y, ws, ws_bytes: int,
                       stream=None) -> None:
    _check(load().ua_prefill_chunked(C.byref(dims), C.byref(params), C.byref(cache), C.byref(tokens), int(n_tokens),
                                     int(chunk), float(log_p), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "ua_prefill_chunked")


def ua_qk_norm(dims, w_q, w_k, eps: float, q, k, n_tokens: int, stream=None) -> None:
    _check(load().ua_qk_norm(C.byref(dims), _ptr(w_q), _ptr(w_k), float(eps), _ptr(q), _ptr(k), int(n_tokens),
                             _stream(stream)), "ua_qk_norm")


def ua_backward_workspace_bytes(dims, n_tokens: int) -> int:
    return int(load().ua_backward_workspace_bytes(C.byref(dims), int(n_tokens)))


def ua_attention_backward(dims, n_tokens: int, q, k, v, lq, lk, lb, dO, dq, dk, dv, dlq, dlk, dlb, ws, ws_bytes: int,
                          stream=None) -> None:
    gi = ua_grad_inputs(*(_ptr(t) for t in (q, k, v, lq, lk, lb, dO)))
    go = ua_grads(*(_ptr(t) for t in (dq, dk, dv, dlq, dlk, dlb)))
    _check(load().ua_attention_backward(C.byref(dims), int(n_tokens), C.byref(gi), C.byref(go), _ptr(ws), ws_bytes,
                                        _stream(stream)), "ua_attention_backward")


def ua_compact(dims, cache, log_p: float, kept_idx, ws, ws_bytes: int, stream=None) -> None:
    _check(load().ua_compact(C.byref(dims), C.byref(cache), float(log_p), _ptr(kept_idx), _ptr(ws), ws_bytes,
                             _stream(stream)), "ua_compact")


def ua_status_string(code: int) -> str:
    return load().ua_status_string(code).decode()


def ua_abi_version() -> int:
    return int(load().ua_abi_version())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_dims(B, H_q, H_kv, d_head, d_model, gate_rank=16, bf16=True, y_bf16=False, terms=UA_TERMS_ALL,
              rope_base=10000.0, sm_scale=0.0) -> ua_dims:
    return ua_dims(B=B, H_q=H_q, H_kv=H_kv, d_head=d_head, d_model=d_model, gate_rank=gate_rank,
                   dtype=UA_BF16 if bf16 else UA_F32, y_dtype=UA_BF16 if y_bf16 else UA_F32, terms=terms,
                   reserved0=0, rope_base=rope_base, sm_scale=sm_scale, reserved1=0.0)


def make_params(W_dec, b_dec, W_dn, W_up, b_up=None) -> ua_params:
    return ua_params(W_dec=_ptr(W_dec), b_dec=_ptr(b_dec), W_dn=_ptr(W_dn), W_up=_ptr(W_up), b_up=_ptr(b_up))


def make_tokens(q, k, v, x) -> ua_tokens:
    return ua_tokens(q=_ptr(q), k=_ptr(k), v=_ptr(v), x=_ptr(x))


def make_cache(K, V, logbias, kgate, seg_off, seg_len, seg_cap, next_pos, status, total_slots=None) -> ua_cache:
    n = K.shape[0] if total_slots is None else total_slots
    return ua_cache(K=_ptr(K), V=_ptr(V), logbias=_ptr(logbias), kgate=_ptr(kgate), seg_off=_ptr(seg_off),
                    seg_len=_ptr(seg_len), seg_cap=_ptr(seg_cap), next_pos=_ptr(next_pos), status=_ptr(status),
                    total_slots=int(n))
