"""Seeded synthetic inputs for the UA layer (shared by tests, bench and smoke).

Holds only random draws and memory layout; none of the layer's arithmetic.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    Weights,
    CacheInit,
    StepInputs,
    bf16_exact,
    bf16_bits,
    make_weights,
    make_cache,
    make_step_inputs,
    make_layout,
    config,
    GradInputs,
    make_grad_inputs,
    MASK_PATTERNS,
    mask_pattern,
    make_mask_cache,
)
