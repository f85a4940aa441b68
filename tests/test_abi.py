"""The C-ABI library loads, exports what include/ua.h declares, sizes its
workspace and rejects bad arguments before touching the GPU (CPU only)."""

import ctypes as C
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ua.h")


def _lib():
    from kv_cache_pruning_amd import _lib as L

    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libua.so not built (run __graft_entry__.build())")
    return L


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(ua_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ua_prefill", "ua_decode_step", "ua_compact", "ua_workspace_bytes", "ua_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    lib = C.CDLL(L.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in include/ua.h but not exported"
    assert set(declared_functions()) == set(L.EXPORTS)


def test_abi_version_and_status_strings():
    L = _lib()
    assert L.ua_abi_version() == 1
    assert L.ua_status_string(0) == "ok"
    assert "workspace" in L.ua_status_string(3)
    assert L.ua_status_string(99) == "unknown status"


def test_struct_layout_matches_header():
    L = _lib()
    assert C.sizeof(L.ua_dims) == 56
    assert L.ua_dims.rope_base.offset == 40
    assert C.sizeof(L.ua_cache) == 80
    assert C.sizeof(L.ua_params) == 40
    assert C.sizeof(L.ua_tokens) == 32
    assert C.sizeof(L.ua_grad_inputs) == 56
    assert C.sizeof(L.ua_grads) == 48


def _dims(L, **kw):
    base = dict(B=8, H_q=32, H_kv=8, d_head=64, d_model=2048, gate_rank=16)
    base.update(kw)
    return L.make_dims(**base)


def test_workspace_bytes():
    L = _lib()
    n1 = L.ua_workspace_bytes(_dims(L), 1, 100_000, 5000)
    n2 = L.ua_workspace_bytes(_dims(L), 1, 200_000, 5000)
    assert n1 > 0 and n2 > n1
    assert L.ua_workspace_bytes(_dims(L, d_head=96), 1, 1000, 100) == 0
    assert L.ua_workspace_bytes(_dims(L, H_q=30), 1, 1000, 100) == 0
    assert L.ua_workspace_bytes(_dims(L), 1, 0, 100) == 0


def _fake_ptr(align=256):
    return 1 << 20  # never dereferenced: every case below fails validation first


def _args(L, **over):
    p = _fake_ptr()
    params = L.ua_params(W_dec=p, b_dec=p, W_dn=p, W_up=p, b_up=None)
    tokens = L.ua_tokens(q=p, k=p, v=p, x=p)
    cache = L.ua_cache(K=p, V=p, logbias=p, kgate=p, seg_off=p, seg_len=p, seg_cap=p, next_pos=p, status=p,
                       total_slots=1000)
    d = dict(params=params, tokens=tokens, cache=cache)
    d.update(over)
    return d


@pytest.mark.parametrize(
    "case,code",
    [
        ("bad_head_dim", 2),
        ("bad_group", 1),
        ("group_5", 2),
        ("nan_log_p", 1),
        ("positive_log_p", 1),
        ("null_y", 1),
        ("misaligned_K", 1),
        ("null_param", 1),
        ("small_ws", 3),
        ("misaligned_ws", 1),
        ("bad_dtype", 1),
        ("terms_8", 1),
    ],
)
def test_decode_step_rejects(case, code):
    L = _lib()
    lib = L.load()
    dims = _dims(L)
    a = _args(L)
    log_p, y, ws, nws = math.log(0.15), _fake_ptr(), _fake_ptr(), 1 << 40
    if case == "bad_head_dim":
        dims = _dims(L, d_head=80)
    elif case == "bad_group":
        dims = _dims(L, H_q=30)
    elif case == "group_5":
        dims = _dims(L, H_q=40)
    elif case == "nan_log_p":
        log_p = float("nan")
    elif case == "positive_log_p":
        log_p = 0.5
    elif case == "null_y":
        y = None
    elif case == "misaligned_K":
        a["cache"].K = _fake_ptr() + 4
    elif case == "null_param":
        a["params"].W_up = None
    elif case == "small_ws":
        nws = 16
    elif case == "misaligned_ws":
        ws = _fake_ptr() + 64
    elif case == "bad_dtype":
        dims.dtype = 7
    elif case == "terms_8":
        dims.terms = 8
    got = lib.ua_decode_step(C.byref(dims), C.byref(a["params"]), C.byref(a["cache"]), C.byref(a["tokens"]), log_p,
                             y, ws, nws, None)
    assert got == code


def test_prefill_and_compact_reject():
    L = _lib()
    lib = L.load()
    a = _args(L)
    p = _fake_ptr()
    assert lib.ua_prefill(C.byref(_dims(L)), C.byref(a["params"]), C.byref(a["cache"]), C.byref(a["tokens"]), 0, p,
                          p, 1 << 40, None) == 1
    assert lib.ua_prefill(C.byref(_dims(L, d_head=32)), C.byref(a["params"]), C.byref(a["cache"]),
                          C.byref(a["tokens"]), 16, p, p, 1 << 40, None) == 2
    assert lib.ua_compact(C.byref(_dims(L)), C.byref(a["cache"]), float("nan"), None, p, 1 << 40, None) == 1
    assert lib.ua_compact(C.byref(_dims(L)), C.byref(a["cache"]), -1.0, p + 2, p, 1 << 40, None) == 1
    assert lib.ua_compact(C.byref(_dims(L)), C.byref(a["cache"]), -1.0, None, p, 8, None) == 3
    bad = _args(L)["cache"]
    bad.seg_len = None
    assert lib.ua_compact(C.byref(_dims(L)), C.byref(bad), -1.0, None, p, 1 << 40, None) == 1


def test_pruned_and_chunked_prefill_reject():
    """Host-side argument checks of the pruned and chunked prefill (no device work)."""
    L = _lib()
    lib = L.load()
    a = _args(L)
    p = _fake_ptr()
    args = (C.byref(_dims(L)), C.byref(a["params"]), C.byref(a["cache"]), C.byref(a["tokens"]))
    assert lib.ua_prefill_pruned(*args, 0, -1.0, p, None, p, 1 << 40, None) == 1       # no tokens
    assert lib.ua_prefill_pruned(*args, 16, float("nan"), p, None, p, 1 << 40, None) == 1
    assert lib.ua_prefill_pruned(*args, 16, 0.5, p, None, p, 1 << 40, None) == 1       # log p > 0
    assert lib.ua_prefill_pruned(*args, 16, -1.0, p, p + 2, p, 1 << 40, None) == 1     # misaligned kept list
    assert lib.ua_prefill_pruned(*args, 16, -1.0, p, None, p, 8, None) == 3            # workspace too small
    assert lib.ua_prefill_chunked(*args, 16, 0, -1.0, p, p, 1 << 40, None) == 1        # empty chunk
    assert lib.ua_prefill_chunked(*args, 0, 8, -1.0, p, p, 1 << 40, None) == 1
    assert lib.ua_prefill_chunked(*args, 16, 8, float("nan"), p, p, 1 << 40, None) == 1
    assert lib.ua_prefill_chunked(*args, 16, 8, -1.0, p, p, 8, None) == 3


def test_varlen_prefill_rejects():
    """Host-side argument checks of ua_prefill_varlen (no device work)."""
    L = _lib()
    lib = L.load()
    a = _args(L)
    p = _fake_ptr()
    args = (C.byref(_dims(L)), C.byref(a["params"]), C.byref(a["cache"]), C.byref(a["tokens"]))
    assert lib.ua_prefill_varlen(*args, None, 10, 8, p, p, 1 << 40, None) == 1      # no offsets
    assert lib.ua_prefill_varlen(*args, p + 2, 10, 8, p, p, 1 << 40, None) == 1     # misaligned offsets
    assert lib.ua_prefill_varlen(*args, p, 0, 8, p, p, 1 << 40, None) == 1          # no rows
    assert lib.ua_prefill_varlen(*args, p, 10, 0, p, p, 1 << 40, None) == 1         # no tokens per sequence
    assert lib.ua_prefill_varlen(*args, p, 10, 8, p, p, 8, None) == 3               # workspace too small


def test_qk_norm_rejects():
    """Host-side argument checks of ua_qk_norm (no device work)."""
    L = _lib()
    lib = L.load()
    p = _fake_ptr()
    d = C.byref(_dims(L))
    assert lib.ua_qk_norm(d, p, p, 1e-6, p, p, 0, None) == 1                # no tokens
    assert lib.ua_qk_norm(d, p, p, float("nan"), p, p, 4, None) == 1
    assert lib.ua_qk_norm(d, p, p, -1.0, p, p, 4, None) == 1
    assert lib.ua_qk_norm(d, p, None, 1e-6, p + 2, p, 4, None) == 1         # misaligned q
    assert lib.ua_qk_norm(d, None, p, 1e-6, p, None, 4, None) == 1          # k weight without k
    assert lib.ua_qk_norm(d, None, None, 1e-6, None, None, 4, None) == 0    # nothing to do
    assert lib.ua_qk_norm(C.byref(_dims(L, d_head=32)), p, p, 1e-6, p, p, 4, None) == 2


def test_attention_backward_rejects():
    """Host-side checks of ua_attention_backward and its workspace size (no device work)."""
    L = _lib()
    lib = L.load()
    p = _fake_ptr()
    d = C.byref(_dims(L))
    assert lib.ua_backward_workspace_bytes(d, 0) == 0
    n = 100
    want = 2 * 64 * n * n * 4 + 2 * 8 * n * 32 * 4  # two N x N fp32 per segment, two [B, N, H_q] vectors
    assert lib.ua_backward_workspace_bytes(d, n) >= want
    gi = L.ua_grad_inputs(*([p] * 7))
    go = L.ua_grads(*([p] * 6))
    ok = lib.ua_backward_workspace_bytes(d, n)
    assert lib.ua_attention_backward(d, 0, C.byref(gi), C.byref(go), p, ok, None) == 1
    assert lib.ua_attention_backward(d, n, C.byref(gi), C.byref(go), p, ok - 1, None) == 3
    bad = L.ua_grad_inputs(*([p] * 6 + [None]))
    assert lib.ua_attention_backward(d, n, C.byref(bad), C.byref(go), p, ok, None) == 1
    bad_do = L.ua_grad_inputs(*([p] * 6 + [p + 4]))  # dO must be 16-byte aligned
    assert lib.ua_attention_backward(d, n, C.byref(bad_do), C.byref(go), p, ok, None) == 1
    bad_out = L.ua_grads(*([p] * 5 + [p + 4]))
    assert lib.ua_attention_backward(d, n, C.byref(gi), C.byref(bad_out), p, ok, None) == 1
    assert lib.ua_attention_backward(C.byref(_dims(L, d_head=32)), n, C.byref(gi), C.byref(go), p, ok, None) == 2


def test_missing_library_fails_loudly(tmp_path):
    from kv_cache_pruning_amd import _lib as L

    with pytest.raises(L.UAError):
        L.load(str(tmp_path / "nope.so"))
