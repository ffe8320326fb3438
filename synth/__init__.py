"""Seeded synthetic inputs for the fused linear + cross-entropy head.

This package only draws random numbers and rounds them to the storage dtype.
It holds none of the loss head's arithmetic, so both the fp64 oracle
(``oracle/``) and the HIP path can be fed from it without sharing any code.
"""

from .configs import CONFIGS, Config, config_by_name
from .generate import (IGNORE, Inputs, make_inputs, make_norm_weight, make_random,
                       mask_preference_rows, to_float64)

__all__ = [
    "CONFIGS",
    "Config",
    "IGNORE",
    "config_by_name",
    "Inputs",
    "make_inputs",
    "make_norm_weight",
    "make_random",
    "mask_preference_rows",
    "to_float64",
]
