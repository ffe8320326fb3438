"""Fused linear + cross-entropy loss head for AMD Instinct MI355X (gfx950).

The work is done by libflce.so (HIP kernels behind the C ABI in
include/flce.h); this package is its Python binding.
"""

from ._lib import (
    CrossEntropyFunction,
    EXPORTS,
    FLCE_BF16,
    FLCE_F32,
    FLCE_STEPS,
    FlceError,
    HipEvents,
    LIB_PATH,
    LinearCrossEntropyFunction,
    STEP_NAMES,
    ce_rows,
    cross_entropy,
    cross_entropy_,
    fwd_bwd,
    fwd_bwd_rmsnorm,
    fwd_bwd_vocab,
    launch_count,
    linear_cross_entropy,
    load,
    logits,
    rmsnorm_workspace_bytes,
    scale_grads,
    vocab_workspace_bytes,
    workspace_bytes,
)

__all__ = [
    "CrossEntropyFunction",
    "EXPORTS",
    "FLCE_BF16",
    "FLCE_F32",
    "FLCE_STEPS",
    "FlceError",
    "HipEvents",
    "LIB_PATH",
    "LinearCrossEntropyFunction",
    "STEP_NAMES",
    "ce_rows",
    "cross_entropy",
    "cross_entropy_",
    "fwd_bwd",
    "fwd_bwd_rmsnorm",
    "fwd_bwd_vocab",
    "launch_count",
    "linear_cross_entropy",
    "load",
    "logits",
    "rmsnorm_workspace_bytes",
    "scale_grads",
    "vocab_workspace_bytes",
    "workspace_bytes",
]
