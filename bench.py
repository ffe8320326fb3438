#!/usr/bin/env python3
"""Throughput of the fused linear + cross-entropy head (forward + backward).

    python bench.py [--gpus 1] [--steps 50] [--warmup 3] [--workload llama3_8b_head]
                    [--chunk C] [--no-cpu-baseline] [--cpu-sample-tokens S]

One step = one flce_fwd_bwd call over the whole batch of the workload
(every token chunk: logits GEMM, row log-sum-exp + gradient rewrite, loss
sum, grad_h GEMM, grad_W GEMM), with inputs already resident in HBM.  The
timed region is bracketed by torch.cuda.synchronize() on both sides.  Prints
one JSON line.

roofline: the dominant kernel (the step with the largest share of GPU time)
timed live with HIP events recorded by flce_fwd_bwd_timed around every
launch, on the stream the kernels run on; achieved = its algorithmic work
per launch (2 * M * N * K flops of one chunk's contraction) / its mean
launch duration.
cpu_baseline: the fp64 CPU oracle on the first S tokens of the same
workload (full V x H head), timed on this host's cores.
mfma_rate: the MFMA rate and shader clock the part sustains running the
GEMMs' instruction stream from registers (flce_mfma_rate), with random and
with zero operands.  pct_measured_mfma_rate relates the step's TFLOP/s to
the random-operand rate.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FLCE fwd+bwd tokens/s + % bf16 MFMA peak; peak workspace bytes"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "llama3_8b_head"
GEMM_STEPS = ("logits_gemm", "grad_h_gemm", "grad_W_gemm")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama3_8b_head.md")
KERNEL_SOURCES = ("gemm_bf16.hip", "gemm_bf16_dma.hip", "ce_rows.hip", "flce_api.hip",
                  "flce_internal.h")


def measure_mfma_rate(flce, torch, dev, iters=40000):
    """The bf16 MFMA rate and shader clock the part sustains for the GEMMs'
    instruction stream with no memory traffic (flce_mfma_rate): one
    256-thread workgroup per CU, 16 32x32x16 MFMAs per round.  It is taken
    once with random operands drawn like the logits GEMM's (N(0,1) by
    N(0, 0.02^2) bf16) and once with zero operands, whose inputs do not
    toggle.  It is timed with events on the current stream."""
    import numpy as np
    wg = torch.cuda.get_device_properties(dev).multi_processor_count
    groups = wg * 4 * 64                      # one 128-byte group per lane
    g = torch.Generator().manual_seed(11)
    a = torch.randn(groups, 32, generator=g)
    b = 0.02 * torch.randn(groups, 32, generator=g)
    cases = {"random": torch.cat([a, b], 1).to(torch.bfloat16).to(dev),
             "zero": torch.zeros(groups, 64, dtype=torch.bfloat16, device=dev)}
    out = {}
    for name, ops in cases.items():
        flce.mfma_rate(ops, iters // 10, wg)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _, clocks = flce.mfma_rate(ops, iters, wg)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        c = clocks.cpu().double().numpy()
        flop = wg * 4.0 * iters * 16 * 32768
        out[name] = {"tflops": flop / (ms * 1e-3) / 1e12,
                     "clock_ghz": float(np.median(c[:, 0] / (c[:, 1] * 10.0))),
                     "ms": ms}
    return {"operands": "bf16, N(0,1) x N(0,0.02^2) (random) and all zero",
            "workgroups": wg, "iters": iters,
            "flop_per_call": wg * 4.0 * iters * 16 * 32768,
            "random_tflops": out["random"]["tflops"],
            "random_clock_ghz": out["random"]["clock_ghz"],
            "zero_tflops": out["zero"]["tflops"],
            "zero_clock_ghz": out["zero"]["clock_ghz"]}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--chunk", type=int, default=0, help="token chunk (default: workload's)")
    p.add_argument("--tokens", type=int, default=0,
                   help="use only the workload's first N tokens (e.g. a ragged last chunk)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=4096)
    p.add_argument("--op", choices=("flce", "ce", "vocab", "rmsnorm", "orpo"), default="flce",
                   help="flce: the fused head (default); ce: cross entropy on given bf16 "
                        "logits [1024, 128256] (flce_cross_entropy); vocab: the fused head "
                        "through flce_fwd_bwd_vocab (vocabulary chunks); rmsnorm: the head "
                        "behind an RMSNorm (flce_fwd_bwd_rmsnorm); orpo: the odds-ratio "
                        "preference loss over the head (flce_orpo_fwd_bwd)")
    p.add_argument("--pairs", type=int, default=4, help="preference pairs of --op orpo")
    p.add_argument("--chunk-pairs", type=int, default=2, help="pairs per chunk of --op orpo")
    p.add_argument("--vchunk", type=int, default=16384,
                   help="vocabulary chunk of --op vocab")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="first run one elementwise fp32 copy of this many MiB (a kernel of "
                        "known traffic, used to scale FETCH_SIZE/WRITE_SIZE counters)")
    return p.parse_args()


def sources_digest() -> str:
    """Digest of the kernel sources' code: comments and whitespace are
    dropped first, so editing a comment does not retire a counter summary."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "linear_cross_entropy_06_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(step: str, workload: str):
    """HBM bytes per launch of `step` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"sources_digest:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != sources_digest():
        return None
    m = re.search(rf"traffic_bytes_per_launch\[{re.escape(workload)}/{re.escape(step)}\]:"
                  rf"\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def cpu_baseline(inp, cfg, sample_tokens: int, chunk: int):
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from synth import to_float64

    S = min(sample_tokens, cfg.N)
    cores = len(os.sched_getaffinity(0))
    blas_threads = max([d.get("num_threads", 0) for d in threadpool_info()] or [cores])
    h64 = to_float64(inp.h[:S])
    W64 = to_float64(inp.W)
    t = inp.t[:S].numpy().astype(np.int64)
    t0 = time.perf_counter()
    loss, _, _ = oracle.flce_chunked(h64, W64, t, chunk)
    dt = time.perf_counter() - t0
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), None)
    except OSError:
        pass
    blas = sorted({f"{d.get('internal_api')} {d.get('version')}" for d in threadpool_info()
                   if d.get("user_api") == "blas"})
    return {
        "value": S / dt,
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "cpu_model": cpu_model,
        "blas": ", ".join(blas) or None,
        "sample": (f"first {S} of {cfg.N} tokens of {cfg.name} against the full "
                   f"{cfg.V}x{cfg.H} head, fp64 numpy oracle, token chunk {chunk}: "
                   f"{dt:.2f} s for {6.0 * S * cfg.V * cfg.H / 1e12:.2f} TFLOP "
                   f"({cores} cores available)"),
    }


def bench_ce(args) -> int:
    """Cross entropy on given logits: p3's [B*S, V] = [1024, 128256] bf16
    logits (std 2, seeded), one flce_cross_entropy call per step (the call
    rewrites the logits in place with their gradient; later steps run on
    that buffer, the same work).  HBM-bound: each call reads the logits
    twice and writes them once."""
    import numpy as np
    import torch

    import linear_cross_entropy_06_amd as flce

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    flce.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    rows, V = 1024, 128256
    g = torch.Generator().manual_seed(args.seed)
    z_cpu = (torch.randn(rows, V, generator=g) * 2.0).to(torch.bfloat16)
    t_cpu = torch.randint(0, V, (rows,), generator=g, dtype=torch.int32)
    z, t = z_cpu.to(dev), t_cpu.to(dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    row_loss = torch.empty(rows, dtype=torch.float32, device=dev)
    first = flce.cross_entropy_(z, t, loss=loss, row_loss=row_loss)
    loss0 = float(first)
    for _ in range(args.warmup):
        flce.cross_entropy_(z, t, loss=loss, row_loss=row_loss)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        flce.cross_entropy_(z, t, loss=loss, row_loss=row_loss)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    bytes_per = rows * V * 2 * 3 + rows * 8
    out = {
        "metric": "cross entropy on given logits: rows/s",
        "value": rows / (ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0, 2^2) logits, uniform targets)",
        "config": {"workload": "ce_on_logits_llama3_vocab", "rows": rows, "V": V},
        "loss_first_call": loss0,
        "roofline": {
            "kernel": "ce_rows_bf16 (+ loss_sum)", "bound": "hbm",
            "achieved": bytes_per / (ev_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": bytes_per / (ev_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
            "work_per_launch": f"{rows}*{V}*2*3 B (logits read twice, written once) "
                               f"= {bytes_per:.4e} B",
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        S = 256
        Z = z_cpu[:S].to(torch.float64).numpy()
        tt = t_cpu[:S].numpy().astype(np.int64)
        c0 = time.perf_counter()
        oracle.row_losses(Z, tt)
        oracle.dlogits(Z, tt, rows)
        dt = time.perf_counter() - c0
        out["cpu_baseline"] = {
            "value": S / dt, "unit": "rows/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"first {S} of {rows} rows, fp64 numpy row_losses + dlogits: {dt:.2f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def bench_vocab(args) -> int:
    """The fused head through flce_fwd_bwd_vocab on a workload (all tokens at
    once, the vocabulary in chunks of --vchunk columns; the logits are formed
    twice, 8 N V H flops, of which 6 N V H are the head's own)."""
    import numpy as np
    import torch

    import linear_cross_entropy_06_amd as flce
    from synth import config_by_name, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    flce.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = config_by_name(args.workload)
    inp = make_inputs(cfg, seed=args.seed)
    h, W, t = inp.h.to(dev), inp.W.to(dev), inp.t.to(dev)
    N, H, V, vc = cfg.N, cfg.H, cfg.V, args.vchunk
    need = flce.vocab_workspace_bytes(N, H, V, vc, h.dtype)
    if need == 0:
        print(f"bench.py: {cfg.name} with vchunk {vc} is not a shape flce_fwd_bwd_vocab runs",
              file=sys.stderr)
        return 1
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    gh = torch.empty_like(h)
    gw = torch.empty((V, H), dtype=torch.float32, device=dev)
    kw = dict(loss=loss, grad_h=gh, grad_W=gw, workspace=ws)
    for _ in range(max(1, args.warmup)):
        flce.fwd_bwd_vocab(h, W, t, vc, **kw)
    torch.cuda.synchronize()
    loss0 = float(loss)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        flce.fwd_bwd_vocab(h, W, t, vc, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    head_flops = 6.0 * N * V * H
    run_flops = 8.0 * N * V * H
    mfma = measure_mfma_rate(flce, torch, h.device)
    out = {
        "metric": "FLCE fwd+bwd tokens/s (vocabulary-chunked entry point)",
        "value": N / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": cfg.name, "N": N, "H": H, "V": V, "vchunk": vc,
                   "seed": args.seed},
        "head_tflops": head_flops / (ms * 1e-3) / 1e12,
        "executed_tflops": run_flops / (ms * 1e-3) / 1e12,
        "pct_measured_mfma_rate": 100.0 * run_flops / (ms * 1e-3) / 1e12 / mfma["random_tflops"],
        "mfma_rate": mfma,
        "workspace_bytes": need,
        "naive_logits_bytes": N * V * 4,
        "token_chunk_workspace_bytes_c4096": flce.workspace_bytes(N, H, V, 4096, h.dtype),
        "loss": loss0,
        "roofline": {
            "kernel": "fwd_bwd_vocab (all launches of one call)", "bound": "mfma",
            "achieved": run_flops / (ev_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": run_flops / (ev_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "traffic": None, "work_per_launch": f"8*{N}*{V}*{H} = {run_flops:.4e} flop",
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        from synth import to_float64
        S = 2048
        hh = to_float64(inp.h[:S])
        WW = to_float64(inp.W)
        tt = inp.t[:S].numpy().astype(np.int64)
        c0 = time.perf_counter()
        oracle.flce_vocab_chunked(hh, WW, tt, vc)
        dt = time.perf_counter() - c0
        out["cpu_baseline"] = {
            "value": S / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"first {S} of {N} tokens against the full {V}x{H} head, fp64 numpy "
                      f"flce_vocab_chunked (vchunk {vc}): {dt:.2f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def bench_rmsnorm(args) -> int:
    """The fused head behind an RMSNorm (flce_fwd_bwd_rmsnorm) on a workload:
    the workload's hidden states are the norm's input x, gamma is a seeded
    weight near 1, eps 1e-6.  Same token chunk as the default bench."""
    import torch

    import linear_cross_entropy_06_amd as flce
    from synth import config_by_name, make_inputs, make_norm_weight

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    flce.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = config_by_name(args.workload)
    inp = make_inputs(cfg, seed=args.seed)
    x, W, t = inp.h.to(dev), inp.W.to(dev), inp.t.to(dev)
    g = make_norm_weight(cfg.H, seed=args.seed).to(dev)
    N, H, V = cfg.N, cfg.H, cfg.V
    C = args.chunk or cfg.default_chunk
    need = flce.rmsnorm_workspace_bytes(N, H, V, C, x.dtype)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    kw = dict(loss=torch.empty((), dtype=torch.float32, device=dev), grad_x=torch.empty_like(x),
              grad_gamma=torch.empty(H, dtype=torch.float32, device=dev),
              grad_W=torch.empty((V, H), dtype=torch.float32, device=dev), workspace=ws)
    for _ in range(max(1, args.warmup)):
        flce.fwd_bwd_rmsnorm(x, g, W, t, C, 1e-6, **kw)
    torch.cuda.synchronize()
    loss0 = float(kw["loss"])
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        flce.fwd_bwd_rmsnorm(x, g, W, t, C, 1e-6, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    flops = 6.0 * N * V * H
    mfma = measure_mfma_rate(flce, torch, x.device)
    out = {
        "metric": "FLCE fwd+bwd tokens/s (behind an RMSNorm, flce_fwd_bwd_rmsnorm)",
        "value": N / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; the workload's hidden states as the norm input)",
        "config": {"workload": cfg.name, "N": N, "H": H, "V": V, "chunk": C, "eps": 1e-6,
                   "seed": args.seed},
        "tflops": flops / (ms * 1e-3) / 1e12,
        "pct_measured_mfma_rate": 100.0 * flops / (ms * 1e-3) / 1e12 / mfma["random_tflops"],
        "mfma_rate": mfma,
        "workspace_bytes": need,
        "loss": loss0,
        "roofline": {
            "kernel": "fwd_bwd_rmsnorm (all launches of one call)", "bound": "mfma",
            "achieved": flops / (ev_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": flops / (ev_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "traffic": None, "work_per_launch": f"6*{N}*{V}*{H} = {flops:.4e} flop",
        },
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_orpo(args) -> int:
    """The odds-ratio preference loss over the head (flce_orpo_fwd_bwd) on a
    workload's head and hidden-state distribution: its N rows read as
    2 * pairs sequences (chosen first) of N / (2 pairs) tokens, each
    sequence's first up-to-256 rows a prompt and last up-to-128 rows padding
    (targets marked ignored), beta 0.1, chunks of --chunk-pairs pairs.  The
    three contractions run over every row: 6 N V H flops a call."""
    import numpy as np
    import torch

    import linear_cross_entropy_06_amd as flce
    from synth import config_by_name, make_inputs, mask_preference_rows

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    flce.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = config_by_name(args.workload)
    N, H, V, B, cp, beta = cfg.N, cfg.H, cfg.V, args.pairs, args.chunk_pairs, 0.1
    if N % (2 * B):
        print(f"bench.py: {N} rows do not split into {2 * B} sequences", file=sys.stderr)
        return 1
    T = N // (2 * B)
    inp = make_inputs(cfg, seed=args.seed)
    t_cpu = mask_preference_rows(inp.t, B, T, seed=args.seed, prompt_max=256, pad_max=128)
    h, W, t = inp.h.to(dev), inp.W.to(dev), t_cpu.to(dev)
    need = flce.orpo_workspace_bytes(B, T, H, V, cp, h.dtype)
    if need == 0:
        print(f"bench.py: {cfg.name} is not a shape flce_orpo_fwd_bwd runs", file=sys.stderr)
        return 1
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    seq = torch.empty(2 * B, dtype=torch.float32, device=dev)
    gh = torch.empty_like(h)
    gw = torch.empty((V, H), dtype=torch.float32, device=dev)
    kw = dict(loss=loss, seq_logp=seq, grad_h=gh, grad_W=gw, workspace=ws)
    for _ in range(max(1, args.warmup)):
        flce.orpo_fwd_bwd(h, W, t, B, T, beta, cp, **kw)
    torch.cuda.synchronize()
    loss0 = float(loss)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        flce.orpo_fwd_bwd(h, W, t, B, T, beta, cp, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    flops = 6.0 * N * V * H
    mfma = measure_mfma_rate(flce, torch, h.device)
    out = {
        "metric": "ORPO over the fused head, fwd+bwd tokens/s",
        "value": N / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; the workload's h, W and targets, prompt and padding "
                "rows marked ignored)",
        "config": {"workload": cfg.name, "N": N, "H": H, "V": V, "pairs": B, "seq_len": T,
                   "chunk_pairs": cp, "beta": beta, "seed": args.seed},
        "counted_rows": int((t_cpu >= 0).sum()),
        "tflops": flops / (ms * 1e-3) / 1e12,
        "pct_measured_mfma_rate": 100.0 * flops / (ms * 1e-3) / 1e12 / mfma["random_tflops"],
        "mfma_rate": mfma,
        "workspace_bytes": need,
        "naive_logits_bytes": N * V * 4,
        "loss": loss0,
        "roofline": {
            "kernel": "orpo_fwd_bwd (all launches of one call)", "bound": "mfma",
            "achieved": flops / (ev_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": flops / (ev_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "traffic": None, "work_per_launch": f"6*{N}*{V}*{H} = {flops:.4e} flop",
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        from synth import to_float64
        S = 512  # one pair of 512-token sequences
        rows = np.r_[0:S, T:T + S]  # first S rows of sequence 0 (chosen) and 1
        hh = to_float64(inp.h[torch.from_numpy(rows)])
        WW = to_float64(inp.W)
        tt = t_cpu[torch.from_numpy(rows)].numpy().astype(np.int64)
        c0 = time.perf_counter()
        oracle.orpo(hh, WW, tt, 1, S, beta)
        dt = time.perf_counter() - c0
        out["cpu_baseline"] = {
            "value": 2 * S / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"one pair of {S}-token sequences (rows of the workload) against the "
                      f"full {V}x{H} head, fp64 numpy orpo: {dt:.2f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    args = parse_args()
    if args.op in ("ce", "vocab", "rmsnorm", "orpo"):
        if args.gpus != 1:
            print("bench.py: this build runs on one GPU only", file=sys.stderr)
            return 2
        return {"ce": bench_ce, "vocab": bench_vocab, "rmsnorm": bench_rmsnorm,
                "orpo": bench_orpo}[args.op](args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the head shards over tokens with one grad_W "
              "all-reduce, which is not part of this build", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import linear_cross_entropy_06_amd as flce
    from synth import config_by_name, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    flce.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = config_by_name(args.workload)
    N, H, V = cfg.N, cfg.H, cfg.V
    if args.tokens:
        if not 1 <= args.tokens <= cfg.N:
            print(f"bench.py: --tokens must lie in [1, {cfg.N}]", file=sys.stderr)
            return 2
        N = args.tokens
    C = args.chunk or cfg.default_chunk or N
    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    t_gen = time.perf_counter()
    inp = make_inputs(cfg, seed=args.seed)
    if N < cfg.N:
        inp = type(inp)(inp.h[:N].contiguous(), inp.W, inp.t[:N].contiguous(), inp.dtype)
    h, W, t = inp.h.to(dev), inp.W.to(dev), inp.t.to(dev)
    t_gen = time.perf_counter() - t_gen

    loss = torch.empty((), dtype=torch.float32, device=dev)
    gh = torch.empty_like(h)
    gw = torch.empty((V, H), dtype=torch.float32, device=dev)
    ws_bytes = flce.workspace_bytes(N, H, V, C, dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    L = flce.launch_count(N, C)
    events = [flce.HipEvents(2 * L) for _ in range(args.steps)]

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.randn(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)   # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        flce.fwd_bwd(h, W, t, C, loss=loss, grad_h=gh, grad_W=gw, workspace=ws)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    mem_before = torch.cuda.max_memory_allocated()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        flce.fwd_bwd(h, W, t, C, loss=loss, grad_h=gh, grad_W=gw, workspace=ws,
                     events=events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    hidden_alloc = torch.cuda.max_memory_allocated() - mem_before

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tok_s = N / (ms_per_step * 1e-3)
    flops = 6.0 * N * V * H
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    # per-step kernel durations from the events
    per_step = {name: [] for name in flce.STEP_NAMES}
    for ev in events:
        for l in range(L):
            per_step[flce.STEP_NAMES[l % flce.FLCE_STEPS]].append(ev.elapsed_ms(2 * l, 2 * l + 1))
    gpu_ms = [ev.elapsed_ms(0, 2 * L - 1) for ev in events]
    for ev in events:
        ev.close()
    avg_ms = {k: float(np.mean(v)) for k, v in per_step.items()}
    tot_ms = {k: float(np.sum(v)) / args.steps for k, v in per_step.items()}
    dominant = max(GEMM_STEPS, key=lambda k: tot_ms[k])
    # rows per launch, averaged over the chunks (C when C divides N)
    rows = N / ((N + C - 1) // C)
    flop_per_launch = 2.0 * rows * V * H
    achieved = flop_per_launch / (avg_ms[dominant] * 1e-3) / 1e12
    traffic = read_traffic(dominant, cfg.name)

    mfma = measure_mfma_rate(flce, torch, dev)

    loss_val = float(loss)
    gold = os.path.join(ROOT, "tests", "golden", f"cfg{cfg.idx}_sampled.npz")
    loss_ref = (float(np.load(gold)["loss"])
                if os.path.exists(gold) and args.seed == 0 and N == cfg.N else None)

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": cfg.name if N == cfg.N else f"{cfg.name} (first {N} tokens)",
                   "N": N, "H": H, "V": V, "chunk": C, "seed": args.seed},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "pct_measured_mfma_rate": 100.0 * tflops / mfma["random_tflops"],
        "mfma_rate": mfma,
        "workspace_bytes": ws_bytes,
        "naive_logits_bytes": N * V * 4,
        "workspace_frac_of_naive": ws_bytes / (N * V * 4),
        "hidden_alloc_bytes": int(hidden_alloc),
        "gpu_ms_per_step_events": float(np.median(gpu_ms)),
        "gpu_ms_per_step_events_min": float(np.min(gpu_ms)),
        "kernel_ms_per_launch": avg_ms,
        "kernel_share": {k: v / sum(tot_ms.values()) for k, v in tot_ms.items()},
        "loss": loss_val,
        "loss_rel_err_vs_oracle": (abs(loss_val - loss_ref) / abs(loss_ref)
                                   if loss_ref else None),
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "work_per_launch": f"2*{rows:g}*{V}*{H} = {flop_per_launch:.4e} flop",
        },
        "input_gen_s": t_gen,
    }
    if not args.no_cpu_baseline:
        del h, W, t, gh, gw, ws
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_sample_tokens, 256)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
