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


def random_shapes(seed: int = 2026, count: int = 32):
    """Seeded (N, H, V, chunk, dtype) cases spread over the shape rules the
    library switches on: H a multiple of 64 or only of 8, V a multiple of 64,
    of 8 or neither, chunks that divide N or leave a ragged last chunk,
    single-row chunks, bf16 and fp32.  Sizes stay small enough for the fp64
    oracle to take about a second a case."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        N = int(np.exp(rng.uniform(0.0, np.log(1500.0))))
        H = 8 * int(rng.integers(1, 65))
        if rng.random() < 0.5:
            H = 64 * max(1, H // 64)
        V = int(np.exp(rng.uniform(0.0, np.log(9000.0))))
        r = rng.random()
        if r < 0.25:
            V = 64 * max(1, V // 64)
        elif r < 0.5:
            V = 8 * max(1, V // 8)
        chunk = int(rng.integers(1, N + 1))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        out.append((max(N, 1), H, max(V, 1), chunk, dtype))
    return out
