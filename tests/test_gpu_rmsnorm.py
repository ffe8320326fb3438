"""GPU parity of flce_fwd_bwd_rmsnorm: the loss head behind an RMSNorm.

x and gamma are the stored inputs of both sides; the oracle
(``oracle.flce_rmsnorm``) normalises them exactly in fp64 and differentiates
by the chain rule, the GPU rounds h and dloss/dh to the storage type once
each.  Small shapes are compared element by element; the full-size
Llama-3-8B head is fed its stored (already RMS-normalised) hidden states
with gamma = 1 and eps = 0, where the norm is the identity up to the
rounding of 1/rms, and compared on sampled rows with the oracle's stored
values plus properties that hold at any size.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs, make_norm_weight, make_random, to_float64
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


SMALL = [
    # N, H, V, chunk, dtype, eps
    (300, 128, 1000, 128, "bf16", 1e-6),   # exponentiated logits path, ragged last chunk
    (512, 256, 768, 256, "bf16", 1e-6),    # every contraction on the direct-to-LDS kernel
    (200, 136, 523, 64, "bf16", 1e-5),     # H % 64 != 0: fp32 logits path
    (17, 64, 1000, 7, "bf16", 0.0),        # eps = 0, tiny chunks
    (100, 64, 333, 33, "f32", 1e-6),       # fp32 operands
    (1024, 512, 8192, 384, "bf16", 1e-6),  # K-split grad_h parts
]


@pytest.mark.parametrize("N,H,V,chunk,dtype,eps", SMALL)
def test_rmsnorm_small(flce, N, H, V, chunk, dtype, eps):
    inp = make_random(N, H, V, dtype=dtype, seed=N + 3 * V, h_std=1.5, w_std=0.3)
    gamma = make_norm_weight(H, dtype=dtype, seed=N)
    x, W, t = to_device(inp)
    g = gamma.cuda()
    say(f"flce_fwd_bwd_rmsnorm N={N} H={H} V={V} chunk={chunk} {dtype} eps={eps}")
    loss, gx, gg, gw = flce.fwd_bwd_rmsnorm(x, g, W, t, chunk, eps)
    torch.cuda.synchronize()
    l0, gx0, gg0, gw0 = oracle.flce_rmsnorm(to_float64(inp.h), to_float64(gamma), eps,
                                            to_float64(inp.W), inp.t.numpy().astype(np.int64))
    el, ex, eg, ew = (rel(float(loss), l0), rel_fro(f64(gx), gx0), rel_fro(f64(gg), gg0),
                      rel_fro(f64(gw), gw0))
    say(f"  loss rel {el:.2e}; grad_x {ex:.2e}; grad_gamma {eg:.2e}; grad_W {ew:.2e}")
    assert el <= LOSS_RTOL and ex <= GRAD_RTOL and eg <= GRAD_RTOL and ew <= GRAD_RTOL


def test_rmsnorm_matches_head_on_normalised_input(flce):
    """The norm's output fed to flce_fwd_bwd gives the same loss and grad_W."""
    N, H, V = 600, 256, 3000
    inp = make_random(N, H, V, dtype="bf16", seed=41, h_std=2.0, w_std=0.1)
    gamma = make_norm_weight(H, seed=41)
    x, W, t = to_device(inp)
    g = gamma.cuda()
    say("rmsnorm vs head on the normalised input")
    loss, gx, gg, gw = flce.fwd_bwd_rmsnorm(x, g, W, t, 256, 1e-6)
    h64, _ = oracle.rmsnorm(to_float64(inp.h), to_float64(gamma), 1e-6)
    h = torch.from_numpy(h64).to(torch.float32).to(torch.bfloat16).cuda()
    l2, gh2, gw2 = flce.fwd_bwd(h, W, t, 256)
    torch.cuda.synchronize()
    assert rel(float(loss), float(l2)) < 1e-4
    assert rel_fro(f64(gw), f64(gw2)) < 5e-3


def test_rmsnorm_gamma_zero_closed_form(flce):
    N, H, V = 300, 128, 1000
    inp = make_random(N, H, V, dtype="bf16", seed=42)
    x, W, t = to_device(inp)
    say("rmsnorm gamma = 0")
    loss, gx, gg, gw = flce.fwd_bwd_rmsnorm(x, torch.zeros(H, dtype=torch.bfloat16,
                                                           device="cuda"), W, t, 128)
    torch.cuda.synchronize()
    assert rel(float(loss), math.log(V)) < 1e-6
    assert torch.count_nonzero(gx).item() == 0
    assert torch.count_nonzero(gw).item() == 0
    _, _, gg0, _ = oracle.flce_rmsnorm(to_float64(inp.h), np.zeros(H), 1e-6, to_float64(inp.W),
                                       inp.t.numpy().astype(np.int64))
    assert rel_fro(f64(gg), gg0) <= GRAD_RTOL


def test_rmsnorm_no_hidden_allocation_and_determinism(flce):
    N, H, V, C = 2048, 1024, 32000, 512
    inp = make_random(N, H, V, dtype="bf16", seed=43)
    x, W, t = to_device(inp)
    g = make_norm_weight(H, seed=43).cuda()
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    gx = torch.empty_like(x)
    gg = torch.empty(H, dtype=torch.float32, device="cuda")
    gw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    need = flce.rmsnorm_workspace_bytes(N, H, V, C, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    kw = dict(loss=loss, grad_x=gx, grad_gamma=gg, grad_W=gw, workspace=ws)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.max_memory_allocated()
    say("rmsnorm no hidden allocation")
    flce.fwd_bwd_rmsnorm(x, g, W, t, C, 1e-6, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base
    first = [v.clone() for v in (loss, gx, gg, gw)]
    flce.fwd_bwd_rmsnorm(x, g, W, t, C, 1e-6, **kw)
    torch.cuda.synchronize()
    for a, b in zip(first, (loss, gx, gg, gw)):
        assert torch.equal(a, b)
    with pytest.raises(flce.FlceError):
        flce.fwd_bwd_rmsnorm(x, g, W, t, C, 1e-6, loss=loss, grad_x=gx, grad_gamma=gg,
                             grad_W=gw, workspace=ws[: need - 16])


def test_rmsnorm_full_size_identity_norm(flce):
    """Llama-3-8B head at the bench's chunk: the stored hidden states are
    already RMS-normalised, so with gamma = 1 and eps = 0 the norm changes
    them only by the rounding of 1/rms.  Loss and sampled rows of grad_W
    against the oracle's stored values; grad_x rows against the chain rule
    applied to the stored grad_h rows; and sum_k grad_x[i, k] x[i, k] = 0
    (the loss does not change along x_i when eps = 0)."""
    cfg = CONFIGS[3]
    p = os.path.join(GOLDEN, "cfg3_sampled.npz")
    if not os.path.exists(p):
        pytest.fail(f"missing {p}: run tests/golden/make_golden.py 3")
    gold = np.load(p, allow_pickle=False)
    say("config 3: generating inputs")
    inp = make_inputs(cfg, seed=0)
    x, W, t = to_device(inp)
    rows = gold["rows"]
    x_rows = to_float64(inp.h[torch.from_numpy(rows)])
    del inp
    H = cfg.H
    g = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    say(f"config 3 fwd_bwd_rmsnorm chunk={cfg.default_chunk}")
    loss, gx, gg, gw = flce.fwd_bwd_rmsnorm(x, g, W, t, cfg.default_chunk, 0.0)
    torch.cuda.synchronize()
    vrows = torch.from_numpy(gold["vocab_rows"]).cuda()
    el = rel(float(loss), float(gold["loss"]))
    ew = rel_fro(f64(gw[vrows]), gold["grad_W_rows"])
    gh = gold["grad_h_rows"]
    r = 1.0 / np.sqrt((x_rows * x_rows).mean(axis=1))
    dot = (gh * x_rows).sum(axis=1)
    gx_exp = r[:, None] * gh - x_rows * (r ** 3 / H * dot)[:, None]
    ex = rel_fro(f64(gx[torch.from_numpy(rows).cuda()]), gx_exp)
    xd = x.double()
    orth = (gx.double() * xd).sum(dim=1).abs().max().item()
    scale = (gx.double().abs() * xd.abs()).sum(dim=1).max().item()
    say(f"  loss rel {el:.2e}; grad_x rows {ex:.2e}; grad_W rows {ew:.2e}; "
        f"max |sum_k grad_x x| {orth:.2e} (sum |.| {scale:.2e})")
    assert el <= LOSS_RTOL and ex <= GRAD_RTOL and ew <= GRAD_RTOL
    assert orth <= 1e-2 * scale
    assert torch.isfinite(gg).all()
