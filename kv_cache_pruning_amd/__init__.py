"""Universal Attention (UA) on MI355X: self-pruning KV cache kernels.

The compute lives in libua.so (hand-written HIP kernels for gfx950 behind a
C ABI, see include/ua.h); this package is its ctypes binding plus a small
device-side container layer (``layer``) over torch tensors.
"""

from ._lib import (  # noqa: F401
    UAError,
    load,
    ua_workspace_bytes,
    ua_workspace_init,
    ua_decode_step,
    ua_decode_compact_step,
    ua_prefill,
    ua_prefill_pruned,
    ua_prefill_chunked,
    ua_prefill_varlen,
    ua_qk_norm,
    ua_backward_workspace_bytes,
    ua_attention_backward,
    ua_compact,
    ua_status_string,
    ua_abi_version,
    make_dims,
    make_params,
    make_tokens,
    make_cache,
)
