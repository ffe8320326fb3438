"""Shared helpers of the GPU parity tests (comparison metrics, device setup).

The tolerances are the parity bar of the loss head on bf16-rounded inputs:
relative error of the loss <= 1e-3, relative Frobenius error of grad_h and
grad_W <= 1e-2, both measured in fp64 against the fp64 oracle run on the
very same stored input values.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

LOSS_RTOL = 1e-3
GRAD_RTOL = 1e-2


def say(*a) -> None:
    """Name the case before a GPU step, flushed, so a fault is attributable."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def rel_fro(a, b) -> float:
    """||a - b||_F / ||b||_F in fp64 (b is the reference)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    d = np.linalg.norm(a - b)
    if nb == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return float(d / nb)


def rel(a: float, b: float) -> float:
    if b == 0.0:
        return abs(a)
    return abs(a - b) / abs(b)


def f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu").to(torch.float64).numpy()


def bf16_rows_from_workspace(z: torch.Tensor, rows: int, V: int) -> np.ndarray:
    """Decode the bf16 gradient rows the row kernel wrote into fp32 rows
    (row i at element offset i * 2 * pitch of the int16 view)."""
    pitch = z.stride(0)
    raw = z.view(torch.int16).reshape(rows, 2 * pitch)[:, :V].contiguous()
    return f64(raw.view(torch.bfloat16))


def to_device(inp, device="cuda"):
    return (inp.h.to(device), inp.W.to(device), inp.t.to(device))
