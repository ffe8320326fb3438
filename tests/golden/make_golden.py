"""Write the oracle's expected values for the full-size workloads.

    python tests/golden/make_golden.py [config ...]      (default: 2 3 4 5)
    python tests/golden/make_golden.py orpo              (preference batch)
    python tests/golden/make_golden.py ragged            (workload 3, 8100 tokens)

Calls only ``synth`` (seeded inputs) and ``oracle`` (fp64 reference).  For
each workload it stores, in ``cfg<k>_sampled.npz``: the mean loss, the
per-row log-sum-exp of every token, sampled token rows (at least one in
every 256-token tile) with their grad_h rows and sampled vocabulary rows (at
least one in every 256-row tile of W) with their grad_W rows (gradients
stored as float32).
"""

from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import (CONFIGS, config_by_name, make_inputs, mask_preference_rows,  # noqa: E402
                   to_float64)

# The preference batch the benchmark times: workload 3's rows as 4 pairs of
# 1024-token sequences, prompts of up to 256 and padding of up to 128 rows
# ignored, beta 0.1.
ORPO = dict(workload="llama3_8b_head", pairs=4, seq_len=1024, prompt_max=256, pad_max=128,
            beta=0.1)


# Output tiles of the GEMMs are 256 x 256: one sampled token row in every
# 256-token tile and one vocabulary row in every 256-row tile of W (the
# last, partial tile included) reach every output tile of grad_h and grad_W.
TILE = 256


def one_per_tile(n: int, rng) -> set:
    return {int(rng.integers(a, min(a + TILE, n))) for a in range(0, n, TILE)}


def sample_rows(cfg, t: np.ndarray):
    """Token rows: one per 256-token tile, both ends, the edges of the
    1024-, 2048- and 4096-token chunks; vocabulary rows: one per 256-row
    tile, both ends, the most frequent target and the targets of the first
    and last token."""
    N, V = cfg.N, cfg.V
    rng = np.random.default_rng([0, 99])
    rows = {0, 1, N // 2, N - 2, N - 1}
    for C in (1024, 2048, 4096, cfg.default_chunk):
        rows |= {min(C - 1, N - 1), min(C, N - 1)}
    rows |= one_per_tile(N, rng)
    vals, counts = np.unique(t, return_counts=True)
    vocab = {0, 1, V // 2, V - 1, int(vals[np.argmax(counts)]), int(t[0]), int(t[N - 1])}
    vocab |= one_per_tile(V, rng)
    return np.array(sorted(rows)), np.array(sorted(vocab))


def make(idx: int) -> str:
    cfg = CONFIGS[idx]
    t0 = time.perf_counter()
    x = make_inputs(cfg, seed=0)
    h, W, t = to_float64(x.h), to_float64(x.W), x.t.numpy().astype(np.int64)
    rows, vocab = sample_rows(cfg, t)
    r = oracle.flce_sampled(h, W, t, rows=rows, vocab_rows=vocab, chunk=1024)
    out = os.path.join(HERE, f"cfg{idx}_sampled.npz")
    np.savez_compressed(
        out,
        config=np.array(cfg.name),
        seed=np.array(0),
        loss=np.array(r["loss"]),
        lse=r["lse"].astype(np.float64),
        rows=rows,
        vocab_rows=vocab,
        grad_h_rows=r["grad_h_rows"].astype(np.float32),
        grad_W_rows=r["grad_W_rows"].astype(np.float32),
    )
    print(f"cfg{idx} {cfg.name}: loss={r['loss']:.9f} rows={len(rows)} "
          f"vocab_rows={len(vocab)} ({time.perf_counter() - t0:.1f} s) -> {out}", flush=True)
    return out


# Workload 3 cut to its first 8100 tokens: at the benchmark's 4096-token
# chunk the last chunk has 4004 rows, so grad_W's contraction length is not
# a multiple of 64 (a partial last slab).
RAGGED = dict(idx=3, N=8100)


def make_ragged() -> str:
    cfg = CONFIGS[RAGGED["idx"]]
    N = RAGGED["N"]
    t0 = time.perf_counter()
    x = make_inputs(cfg, seed=0)
    h, W, t = to_float64(x.h[:N]), to_float64(x.W), x.t[:N].numpy().astype(np.int64)
    V = cfg.V
    rng = np.random.default_rng([0, 97])
    rows = {0, N - 1, 4095, 4096, 4097, N - 2} | one_per_tile(N, rng)
    # every 4th 256-row tile of W, the last one included, and the targets of
    # the last chunk's first and last token
    vocab = {int(rng.integers(a, min(a + TILE, V))) for a in range(0, V, 4 * TILE)}
    vocab |= {V - 1, int(t[4096]), int(t[N - 1])}
    rows, vocab = np.array(sorted(rows)), np.array(sorted(vocab))
    r = oracle.flce_sampled(h, W, t, rows=rows, vocab_rows=vocab, chunk=1024)
    out = os.path.join(HERE, f"cfg{RAGGED['idx']}_n{N}_sampled.npz")
    np.savez_compressed(
        out,
        config=np.array(cfg.name),
        seed=np.array(0),
        tokens=np.array(N),
        loss=np.array(r["loss"]),
        rows=rows,
        vocab_rows=vocab,
        grad_h_rows=r["grad_h_rows"].astype(np.float32),
        grad_W_rows=r["grad_W_rows"].astype(np.float32),
    )
    print(f"cfg{RAGGED['idx']} first {N} tokens: loss={r['loss']:.9f} rows={len(rows)} "
          f"vocab_rows={len(vocab)} ({time.perf_counter() - t0:.1f} s) -> {out}", flush=True)
    return out


def make_orpo() -> str:
    cfg = config_by_name(ORPO["workload"])
    B, T = ORPO["pairs"], ORPO["seq_len"]
    t0 = time.perf_counter()
    x = make_inputs(cfg, seed=0)
    tm = mask_preference_rows(x.t, B, T, seed=0, prompt_max=ORPO["prompt_max"],
                              pad_max=ORPO["pad_max"])
    h, W, t = to_float64(x.h), to_float64(x.W), tm.numpy().astype(np.int64)
    N, V = cfg.N, cfg.V
    rng = np.random.default_rng([0, 98])
    # sequence starts and ends, the chunk boundary of 2-pair chunks, a prompt
    # row (ignored), the last counted row of a sequence, a few random rows
    rows = {0, T - 1, T, 2 * T - 1, B * T - 1, B * T, N - 1, 2 * T, 2 * T * B // 2}
    rows |= {int(np.nonzero(t < 0)[0][0]), int(np.nonzero(t[:T] >= 0)[0][-1])}
    rows |= set(rng.integers(0, N, 5).tolist())
    rows |= one_per_tile(N, rng)
    rows = np.array(sorted(rows))
    vals, counts = np.unique(t[t >= 0], return_counts=True)
    vocab = {0, 1, V // 2, V - 1, int(vals[np.argmax(counts)])}
    vocab |= {int(t[r]) for r in rows[:16] if t[r] >= 0}
    vocab |= set(rng.integers(0, V, 4).tolist())
    vocab |= one_per_tile(V, rng)
    vocab = np.array(sorted(vocab))
    r = oracle.orpo_sampled(h, W, t, B, T, ORPO["beta"], rows=rows, vocab_rows=vocab,
                            chunk=1024)
    out = os.path.join(HERE, "orpo_llama3_8b_head_sampled.npz")
    np.savez_compressed(
        out,
        config=np.array(cfg.name),
        seed=np.array(0),
        pairs=np.array(B),
        seq_len=np.array(T),
        prompt_max=np.array(ORPO["prompt_max"]),
        pad_max=np.array(ORPO["pad_max"]),
        beta=np.array(ORPO["beta"]),
        loss=np.array(r["loss"]),
        seq_logp=r["seq_logp"],
        rows=rows,
        vocab_rows=vocab,
        grad_h_rows=r["grad_h_rows"].astype(np.float32),
        grad_W_rows=r["grad_W_rows"].astype(np.float32),
    )
    print(f"orpo {cfg.name}: loss={r['loss']:.9f} rows={len(rows)} vocab_rows={len(vocab)} "
          f"({time.perf_counter() - t0:.1f} s) -> {out}", flush=True)
    return out


if __name__ == "__main__":
    args = sys.argv[1:] or ["2", "3", "4", "5"]
    for a in args:
        if a == "orpo":
            make_orpo()
        elif a == "ragged":
            make_ragged()
        else:
            make(int(a))
