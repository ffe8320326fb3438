"""GPU parity of the vocabulary-chunked entry point, flce_fwd_bwd_vocab.

All tokens at once, the vocabulary in column chunks: a statistics pass over
every chunk, then the gradients chunk by chunk with the global log-sum-exp.
The result is the same loss head, so it is compared with the fp64 oracle
(the plain definition, and its vocabulary-chunked form) on the same stored
inputs, with the token-chunked entry point, and on sampled rows of the
full-size workloads against the stored oracle values.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs, make_random, to_float64
from parity_util import GRAD_RTOL, LOSS_RTOL, f64, rel, rel_fro, say, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def flce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_06_amd as m
    m.load()  # raises if the HIP library is missing: no fallback exists
    return m


def _check(name, got, exp):
    loss, gh, gw = got
    l0, gh0, gw0 = exp
    el, eh, ew = rel(float(loss), l0), rel_fro(f64(gh), gh0), rel_fro(f64(gw), gw0)
    say(f"{name}: loss {float(loss):.7f} vs {l0:.7f} rel {el:.2e}; "
        f"grad_h rel_fro {eh:.2e}; grad_W rel_fro {ew:.2e}")
    assert np.isfinite(float(loss))
    assert el <= LOSS_RTOL and eh <= GRAD_RTOL and ew <= GRAD_RTOL, (name, el, eh, ew)


SMALL = [
    # N, H, V, vchunk
    (300, 128, 1024, 256),    # 4 chunks; 300 tokens: grad_W's K = N off the 64-multiple kernel
    (512, 256, 2048, 512),    # every contraction on the direct-to-LDS kernel
    (200, 64, 1664, 512),     # last chunk 128 columns
    (64, 64, 40000, 4096),    # ten chunks, the last 3136 columns
    (1, 64, 256, 128),        # one token
    (257, 192, 768, 10 ** 6),  # one chunk (vchunk >= V)
]


@pytest.mark.parametrize("N,H,V,vchunk", SMALL)
def test_vocab_small(flce, N, H, V, vchunk):
    inp = make_random(N, H, V, dtype="bf16", seed=N * 7 + V, w_std=0.3)
    h, W, t = to_device(inp)
    say(f"flce_fwd_bwd_vocab N={N} H={H} V={V} vchunk={vchunk}")
    got = flce.fwd_bwd_vocab(h, W, t, vchunk)
    torch.cuda.synchronize()
    hh, WW, tt = to_float64(inp.h), to_float64(inp.W), inp.t.numpy().astype(np.int64)
    exp = oracle.flce_vocab_chunked(hh, WW, tt, min(vchunk, V))
    _check(f"vocab{(N, H, V, vchunk)}", got, exp)


def test_vocab_matches_token_chunked_and_is_deterministic(flce):
    N, H, V = 1024, 256, 4096
    inp = make_random(N, H, V, dtype="bf16", seed=31, w_std=0.1)
    h, W, t = to_device(inp)
    say("vocab vs token-chunked")
    a = tuple(x.clone() for x in flce.fwd_bwd_vocab(h, W, t, 1024))
    b = flce.fwd_bwd(h, W, t, 256)
    torch.cuda.synchronize()
    assert rel(float(a[0]), float(b[0])) < 1e-5
    assert rel_fro(f64(a[1]), f64(b[1])) < 5e-3
    assert rel_fro(f64(a[2]), f64(b[2])) < 5e-3
    say("vocab determinism")
    again = flce.fwd_bwd_vocab(h, W, t, 1024)
    torch.cuda.synchronize()
    for x, y in zip(a, again):
        assert torch.equal(x, y)
    # other chunk widths agree to rounding
    c = flce.fwd_bwd_vocab(h, W, t, 384)
    torch.cuda.synchronize()
    assert rel(float(c[0]), float(a[0])) < 1e-5
    assert rel_fro(f64(c[2]), f64(a[2])) < 2e-3


def test_vocab_closed_form_w_zero(flce):
    N, H, V = 300, 64, 1024
    inp = make_random(N, H, V, dtype="bf16", seed=32)
    h, W, t = to_device(inp)
    say("vocab W = 0 closed form")
    loss, gh, gw = flce.fwd_bwd_vocab(h, torch.zeros_like(W), t, 256)
    torch.cuda.synchronize()
    assert rel(float(loss), math.log(V)) < 1e-6
    assert torch.count_nonzero(gh).item() == 0
    hh = to_float64(inp.h)
    exp_gw = np.tile(hh.sum(axis=0) / V, (V, 1))
    np.add.at(exp_gw, inp.t.numpy(), -hh)
    assert rel_fro(f64(gw), exp_gw / N) < GRAD_RTOL


def test_vocab_no_hidden_allocation(flce):
    N, H, V, vc = 2048, 1024, 32000, 8192
    inp = make_random(N, H, V, dtype="bf16", seed=33)
    h, W, t = to_device(inp)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    gh = torch.empty_like(h)
    gw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    need = flce.vocab_workspace_bytes(N, H, V, vc, torch.bfloat16)
    rup = lambda x: (x + 255) // 256 * 256
    # bf16 logits of a chunk, pairs, 4 floats per row, fp32 grad_h accumulator
    assert need == rup(rup(rup(N * vc * 2) + N * ((V + 127) // 128) * 8) + 4 * N * 4) + N * H * 4
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.max_memory_allocated()
    say("vocab no hidden allocation")
    flce.fwd_bwd_vocab(h, W, t, vc, loss=loss, grad_h=gh, grad_W=gw, workspace=ws)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base
    with pytest.raises(flce.FlceError):
        flce.fwd_bwd_vocab(h, W, t, vc, loss=loss, grad_h=gh, grad_W=gw,
                           workspace=ws[: need - 16])


def test_vocab_out_of_range_target_is_nan(flce):
    inp = make_random(8, 64, 256, dtype="bf16", seed=34)
    h, W, t = to_device(inp)
    t[3] = 256
    say("vocab out-of-range target")
    loss, gh, gw = flce.fwd_bwd_vocab(h, W, t, 128)
    torch.cuda.synchronize()
    assert math.isnan(float(loss))


VOCAB_CHUNK = {3: 16384, 5: 32768}


@pytest.mark.parametrize("idx", [3, 5])
def test_vocab_full_size_sampled(flce, idx):
    """Full-size workloads through the vocabulary-chunked path: loss and
    sampled rows against the oracle's stored values, plus sum_j grad_W = 0."""
    cfg = CONFIGS[idx]
    p = os.path.join(GOLDEN, f"cfg{idx}_sampled.npz")
    if not os.path.exists(p):
        pytest.fail(f"missing {p}: run tests/golden/make_golden.py {idx}")
    gold = np.load(p, allow_pickle=False)
    say(f"config {idx} ({cfg.name}): generating inputs")
    inp = make_inputs(cfg, seed=0)
    h, W, t = to_device(inp)
    del inp
    vc = VOCAB_CHUNK[idx]
    say(f"config {idx} fwd_bwd_vocab vchunk={vc}")
    loss, gh, gw = flce.fwd_bwd_vocab(h, W, t, vc)
    torch.cuda.synchronize()
    rows = torch.from_numpy(gold["rows"]).cuda()
    vrows = torch.from_numpy(gold["vocab_rows"]).cuda()
    el = rel(float(loss), float(gold["loss"]))
    eh = rel_fro(f64(gh[rows]), gold["grad_h_rows"])
    ew = rel_fro(f64(gw[vrows]), gold["grad_W_rows"])
    colsum = gw.double().sum(dim=0).abs().max().item()
    scale = gw.double().abs().sum(dim=0).max().item()
    say(f"  loss {float(loss):.6f} vs {float(gold['loss']):.6f} rel {el:.2e}; "
        f"grad_h rows rel_fro {eh:.2e}; grad_W rows rel_fro {ew:.2e}; "
        f"|sum_j grad_W| {colsum:.2e} (sum |.| {scale:.2e})")
    assert el <= LOSS_RTOL and eh <= GRAD_RTOL and ew <= GRAD_RTOL
    assert colsum <= 1e-3 * scale
