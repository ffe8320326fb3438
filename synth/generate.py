"""Seeded generation of (h, W, targets) for the loss head.

Recipe (every step is fixed, so that every machine sees identical bits):

* Every tensor is drawn in blocks of ``BLOCK_ROWS`` rows.  Block ``b`` of the
  tensor with tag ``T`` uses its own PCG64 stream,
  ``numpy.random.default_rng([seed, T, b])``; tags are h=1, W=2, targets=3,
  outlier positions=4 (a norm weight, ``make_norm_weight``, draws on
  ``[seed, 5]``; the prompt and padding lengths of a preference batch,
  ``mask_preference_rows``, on ``[seed, 6]``).  Blocks are independent, so they are drawn in threads.
* h: ``standard_normal`` in fp64.  ``rms_normal`` then divides each row by
  ``sqrt(mean(row**2) + 1e-6)`` (the output of an RMS norm with unit gain);
  ``normal_outliers`` multiplies ``round(0.001 * N * H)`` distinct entries,
  chosen with ``choice(N*H, K, replace=False)`` on stream ``[seed, 4]``, by 20.
* W: ``0.02 * standard_normal`` in fp64.
* targets (int32): ``uniform`` is ``integers(0, V, N)`` on stream
  ``[seed, 3]``; ``zipf`` draws rank k in [0, V) with probability
  proportional to ``(k + 1) ** -1.1`` by inverse CDF (``searchsorted`` of the
  fp64 cumulative weights against ``random(N)`` on stream ``[seed, 3]``),
  and rank k is token id k.
* Rounding: fp64 -> fp32 (round to nearest even); for bf16 workloads then
  fp32 -> bf16 (round to nearest even, torch's CPU cast).  These stored bits
  are the inputs of both the HIP path and the oracle; the oracle upcasts them
  exactly.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

from .configs import Config

BLOCK_ROWS = 1024
TAG_H, TAG_W, TAG_T, TAG_OUTLIER = 1, 2, 3, 4


@dataclass
class Inputs:
    h: torch.Tensor        # [N, H] bf16 or fp32, CPU
    W: torch.Tensor        # [V, H] bf16 or fp32, CPU
    t: torch.Tensor        # [N] int32, CPU
    dtype: str             # "bf16" | "f32"

    @property
    def N(self) -> int:
        return self.h.shape[0]

    @property
    def H(self) -> int:
        return self.h.shape[1]

    @property
    def V(self) -> int:
        return self.W.shape[0]


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_blocks(seed: int, tag: int, rows: int, cols: int, scale: float,
                 dtype: str, transform=None) -> torch.Tensor:
    """Draw a [rows, cols] normal tensor block by block into the storage dtype."""
    out = torch.empty((rows, cols), dtype=_torch_dtype(dtype))
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def one(b: int) -> None:
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        rng = np.random.default_rng([seed, tag, b])
        x = rng.standard_normal((r1 - r0, cols))
        if scale != 1.0:
            x *= scale
        if transform is not None:
            x = transform(x, r0)
        out[r0:r1] = torch.from_numpy(x.astype(np.float32))

    if nblk == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nblk)))
    return out


def _targets(seed: int, N: int, V: int, kind: str, zipf_s: float) -> torch.Tensor:
    rng = np.random.default_rng([seed, TAG_T])
    if kind == "uniform":
        t = rng.integers(0, V, N, dtype=np.int32)
    elif kind == "zipf":
        w = np.arange(1, V + 1, dtype=np.float64) ** (-zipf_s)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        u = rng.random(N)
        t = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int32)
    else:
        raise ValueError(f"unknown target distribution {kind!r}")
    return torch.from_numpy(t)


def make_inputs(cfg: Config, seed: int = 0) -> Inputs:
    """The workload ``cfg`` as CPU tensors in its storage dtype."""
    N, H, V = cfg.N, cfg.H, cfg.V
    transform = None
    if cfg.h_dist == "rms_normal":
        eps = cfg.rms_eps

        def transform(x, r0):
            return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    elif cfg.h_dist == "normal_outliers":
        K = int(round(cfg.outlier_frac * N * H))
        pos = np.random.default_rng([seed, TAG_OUTLIER]).choice(N * H, K, replace=False)
        pos.sort()
        scale = cfg.outlier_scale

        def transform(x, r0):
            lo, hi = r0 * H, (r0 + x.shape[0]) * H
            a, b = np.searchsorted(pos, [lo, hi])
            flat = x.reshape(-1)
            flat[pos[a:b] - lo] *= scale
            return x
    elif cfg.h_dist != "normal":
        raise ValueError(cfg.h_dist)
    h = _draw_blocks(seed, TAG_H, N, H, 1.0, cfg.dtype, transform)
    W = _draw_blocks(seed, TAG_W, V, H, cfg.w_std, cfg.dtype)
    t = _targets(seed, N, V, cfg.targets, cfg.zipf_s)
    return Inputs(h=h, W=W, t=t, dtype=cfg.dtype)


def make_random(N: int, H: int, V: int, dtype: str = "bf16", seed: int = 0,
                h_std: float = 1.0, w_std: float = 0.02,
                targets: str = "uniform") -> Inputs:
    """A small workload of arbitrary shape (edge cases, ragged tails)."""
    h = _draw_blocks(seed, TAG_H, N, H, h_std, dtype)
    W = _draw_blocks(seed, TAG_W, V, H, w_std, dtype)
    t = _targets(seed, N, V, targets, 1.1)
    return Inputs(h=h, W=W, t=t, dtype=dtype)


TAG_GAMMA = 5


def make_norm_weight(H: int, dtype: str = "bf16", seed: int = 0, std: float = 0.1) -> torch.Tensor:
    """A norm weight [H] near 1: ``1 + std * standard_normal`` on stream
    ``[seed, 5]``, rounded like every other input (fp64 -> fp32 -> bf16)."""
    x = 1.0 + std * np.random.default_rng([seed, TAG_GAMMA]).standard_normal(H)
    t = torch.from_numpy(x.astype(np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_float64(x: torch.Tensor) -> np.ndarray:
    """Exact upcast of stored bf16/fp32 values to fp64 numpy."""
    return x.detach().to("cpu").to(torch.float64).numpy()


TAG_MASK = 6
IGNORE = -100


def mask_preference_rows(t: torch.Tensor, pairs: int, seq_len: int, seed: int = 0,
                         prompt_max: int = 0, pad_max: int = 0) -> torch.Tensor:
    """Targets of a preference batch (2 * pairs sequences of seq_len rows,
    chosen responses first) with prompt and padding rows marked IGNORE.

    On stream ``[seed, 6]``: per pair a prompt length ``integers(0,
    prompt_max + 1)`` shared by its two sequences, then per sequence (chosen
    of every pair, then rejected) a padding length ``integers(0, pad_max +
    1)``; both are cut so that every sequence keeps at least one row.  The
    first prompt-length rows and the last padding-length rows of each
    sequence become IGNORE."""
    rng = np.random.default_rng([seed, TAG_MASK])
    prompt = rng.integers(0, prompt_max + 1, pairs)
    pad = rng.integers(0, pad_max + 1, 2 * pairs)
    out = t.clone()
    v = out.view(2 * pairs, seq_len)
    for s in range(2 * pairs):
        a = min(int(prompt[s % pairs]), seq_len - 1)
        b = min(int(pad[s]), seq_len - 1 - a)
        v[s, :a] = IGNORE
        if b > 0:
            v[s, seq_len - b:] = IGNORE
    return out
