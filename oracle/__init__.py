"""Plain fp64 CPU oracle for Universal Attention (UA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP path (no kernels, headers, helpers, tables or pre/post-processing) and does
not import the generators; callers pass plain numpy arrays in.

Source of the method: "A Self-Pruning Transformer: Extreme KV-Cache Compression
with Universal Attention" as summarised on the paperlayer.ai page (sections 3,
4, 4.1, 4.2, App. C) and the ai4snews page (Figure 1 caption and the paragraphs
after it).  ``ua_ref`` holds the specification and its readings.
"""

from .ua_ref import (  # noqa: F401
    Dims,
    Params,
    RefCache,
    TERM_Q,
    TERM_K,
    TERM_SIM,
    TERMS_ALL,
    bf16_round,
    round_cache,
    sigmoid,
    l2_normalize,
    qk_rmsnorm,
    rope,
    log_sigmoid,
    log1mexp,
    gates,
    output_gate,
    pair_term,
    attend,
    preprocess_token,
    decode_step,
    prefill,
    prefill_varlen,
    compact,
    dense_logbias,
    dense_attention,
)

from . import ua_grad  # noqa: F401,E402  (torch fp64 autograd reference for the backward pass)
