"""fp64 CPU oracle of the fused linear + cross-entropy head.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously correct
reference the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path (``linear_cross_entropy_06_amd``) never does and
shares no code with it.
"""

from .flce_oracle import (
    dlogits,
    flce,
    flce_brute,
    flce_chunked,
    flce_rmsnorm,
    flce_sampled,
    flce_vocab_chunked,
    logits,
    logsumexp_rows,
    rmsnorm,
    row_losses,
)
from .orpo_oracle import orpo, orpo_sampled, token_logp

__all__ = [
    "dlogits",
    "flce",
    "flce_brute",
    "flce_chunked",
    "flce_rmsnorm",
    "flce_sampled",
    "flce_vocab_chunked",
    "logits",
    "logsumexp_rows",
    "orpo",
    "orpo_sampled",
    "rmsnorm",
    "row_losses",
    "token_logp",
]
