"""GPU parity of flce_orpo_fwd_bwd: the odds-ratio preference loss over the
fused head, against the fp64 oracle ``oracle.orpo`` on the same stored
inputs (bf16 h and W, int32 targets with prompt and padding rows marked
negative), element by element, plus closed forms and properties of the
GPU result itself.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import IGNORE, make_random, mask_preference_rows, to_float64
from parity_util import GRAD_RTOL, LOSS_RTOL, f64, rel, rel_fro, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def flce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_06_amd as m
    m.load()  # raises if the HIP library is missing: no fallback exists
    return m


def _inputs(B, T, H, V, seed, prompt_max, pad_max, w_std=0.3):
    inp = make_random(2 * B * T, H, V, dtype="bf16", seed=seed, w_std=w_std)
    t = mask_preference_rows(inp.t, B, T, seed=seed, prompt_max=prompt_max, pad_max=pad_max)
    return inp.h, inp.W, t


def _oracle(h, W, t, B, T, beta):
    return oracle.orpo(to_float64(h), to_float64(W), t.numpy().astype(np.int64), B, T, beta)


def _check(name, got, exp, seq_rtol=1e-4):
    loss, seq, gh, gw = got
    l0, gh0, gw0, seq0 = exp
    el, eh, ew = rel(float(loss), l0), rel_fro(f64(gh), gh0), rel_fro(f64(gw), gw0)
    es = float(np.max(np.abs(f64(seq) - seq0) / np.maximum(np.abs(seq0), 1e-3)))
    say(f"{name}: loss {float(loss):.7f} vs {l0:.7f} rel {el:.2e}; seq_logp {es:.2e}; "
        f"grad_h {eh:.2e}; grad_W {ew:.2e}")
    assert np.isfinite(float(loss))
    assert el <= LOSS_RTOL and es <= seq_rtol and eh <= GRAD_RTOL and ew <= GRAD_RTOL, \
        (name, el, es, eh, ew)


SMALL = [
    # pairs, seq_len, H, V, chunk_pairs, beta, prompt_max, pad_max
    (2, 8, 64, 256, 1, 0.1, 3, 2),          # one pair per chunk
    (3, 50, 128, 1000, 2, 1.0, 10, 5),      # ragged last chunk; V % 64 != 0
    (4, 64, 256, 2048, 4, 0.5, 16, 8),      # one chunk, every contraction on the LDS-DMA kernel
    (2, 300, 128, 1024, 1, 5.0, 40, 20),    # large beta
    (1, 1, 64, 256, 1, 0.1, 0, 0),          # one token per sequence
    (8, 128, 512, 4096, 3, 0.1, 32, 16),    # K-split grad_h parts, ragged chunks
]


@pytest.mark.parametrize("B,T,H,V,cp,beta,pm,pd", SMALL)
def test_orpo_small(flce, B, T, H, V, cp, beta, pm, pd):
    h, W, t = _inputs(B, T, H, V, seed=B * 31 + T, prompt_max=pm, pad_max=pd)
    hd, Wd, td = h.cuda(), W.cuda(), t.cuda()
    say(f"flce_orpo_fwd_bwd pairs={B} seq_len={T} H={H} V={V} chunk_pairs={cp} beta={beta}")
    got = flce.orpo_fwd_bwd(hd, Wd, td, B, T, beta, cp)
    torch.cuda.synchronize()
    _check(f"orpo{(B, T, H, V, cp, beta)}", got, _oracle(h, W, t, B, T, beta))


def test_orpo_confident_model(flce):
    """Hidden states aligned with their targets' weight rows: p(target) near
    1, mean log-probabilities near 0, where 1 - exp(l) needs care."""
    B, T, H, V = 2, 16, 128, 512
    inp = make_random(2 * B * T, H, V, dtype="bf16", seed=51, w_std=0.3)
    t = mask_preference_rows(inp.t, B, T, seed=51, prompt_max=3, pad_max=2)
    W = inp.W.float()
    tt = t.clamp(min=0).long()
    h = (W[tt] + 0.05 * inp.h.float()).to(torch.bfloat16)
    say("orpo confident model")
    got = flce.orpo_fwd_bwd(h.cuda(), inp.W.cuda(), t.cuda(), B, T, 0.5, 1)
    torch.cuda.synchronize()
    exp = _oracle(h, inp.W, t, B, T, 0.5)
    assert float(np.min(exp[3])) > -0.1  # the case is what it claims to be: p ~ 0.97-0.99
    _check("orpo confident", got, exp, seq_rtol=2e-3)


def test_orpo_certain_sequences(flce):
    """Two-valued logits (W = I, a counted row h = m e_t: logit m at the
    target, 0 elsewhere).  Pair 0 has a certain chosen sequence (margin 40:
    1 - p ~ 1e-15) and pair 1 a certain rejected one: finite loss and
    gradients equal to the oracle's, and each sequence's mean
    log-probability (about -2.3e-15 for the certain ones) to its relative
    precision: the mass of the other classes comes from fp32 sums, except
    in the target's own 128-column slice, whose exponentials are stored in
    bf16 (here all 127 round the same way: at most 2^-9 on half of S)."""
    B, T, H, V, beta = 2, 8, 256, 256, 0.5
    _, _, t = _inputs(B, T, H, V, seed=58, prompt_max=2, pad_max=1)
    W = torch.eye(V, H).to(torch.bfloat16)
    margin = [40.0, 10.0, 10.0, 40.0]  # chosen 0, chosen 1, rejected 0, rejected 1
    h = torch.zeros(2 * B * T, H)
    for r in range(2 * B * T):
        if t[r] >= 0:
            h[r, int(t[r])] = margin[r // T]
    h = h.to(torch.bfloat16)
    say("orpo certain sequences")
    got = flce.orpo_fwd_bwd(h.cuda(), W.cuda(), t.cuda(), B, T, beta, 1)
    torch.cuda.synchronize()
    exp = _oracle(h, W, t, B, T, beta)
    assert -1e-14 < exp[3][0] < 0.0 and -1e-14 < exp[3][3] < 0.0  # certain, and still < 0
    assert all(torch.isfinite(x).all() for x in got)
    es = float(np.max(np.abs(f64(got[1]) / exp[3] - 1.0)))
    say(f"  seq_logp relative error {es:.2e}")
    assert es <= 2e-3
    _check("orpo certain", got, exp, seq_rtol=2e-3)


def _confident_h(W, t, noise, level, rows):
    """h for the given rows: kappa W[t] + 0.05 noise, kappa chosen so the
    rows' mean log-probability (fp64, bf16-rounded h) is near `level`."""
    Wd = W.double()
    tt = t[rows].clamp(min=0).long()
    counted = (t[rows] >= 0).numpy()

    def mean_logp(kappa):
        hh = (kappa * W[tt].float() + 0.05 * noise[rows].float()).to(torch.bfloat16).double()
        Z = (hh @ Wd.T).numpy()
        zt = Z[np.arange(len(rows)), tt.numpy()]
        D = Z - zt[:, None]
        D[np.arange(len(rows)), tt.numpy()] = -np.inf
        return float(np.mean(-np.log1p(np.exp(D).sum(axis=1))[counted])), hh

    lo, hi = 0.05, 10.0  # mean log p rises towards 0 as kappa grows
    for _ in range(50):
        mid = 0.5 * (lo + hi)
        if mean_logp(mid)[0] < level:
            lo = mid
        else:
            hi = mid
    return mean_logp(0.5 * (lo + hi))[1]


@pytest.mark.parametrize("lw,ll", [(-1e-4, -3e-4), (-3e-4, -1e-3), (-1e-3, -1e-4)])
def test_orpo_confident_levels(flce, lw, ll):
    """Mean log-probabilities of 1e-4 to 1e-3 below 0, where 1 - exp(l) is
    what the odds divide by: loss, gradients and every sequence's mean
    log-probability against the oracle at the usual tolerances."""
    B, T, H, V, beta = 2, 64, 256, 512, 0.5
    inp = make_random(2 * B * T, H, V, dtype="bf16", seed=60, w_std=0.3)
    t = mask_preference_rows(inp.t, B, T, seed=60, prompt_max=8, pad_max=4)
    h = torch.zeros(2 * B * T, H, dtype=torch.float64)
    levels = [lw] * B + [ll] * B
    for s_ in range(2 * B):
        rows = torch.arange(s_ * T, (s_ + 1) * T)
        h[rows] = _confident_h(inp.W, t, inp.h, levels[s_], rows)
    h = h.to(torch.bfloat16)
    say(f"orpo confident levels {lw} / {ll}")
    got = flce.orpo_fwd_bwd(h.cuda(), inp.W.cuda(), t.cuda(), B, T, beta, 1)
    torch.cuda.synchronize()
    exp = _oracle(h, inp.W, t, B, T, beta)
    lv = np.array(levels)
    assert np.all((exp[3] / lv > 0.8) & (exp[3] / lv < 1.25)), exp[3]  # the case is as named
    es = float(np.max(np.abs(f64(got[1]) / exp[3] - 1.0)))
    say(f"  seq_logp relative error {es:.2e}")
    assert es <= 1e-3
    _check(f"orpo confident {lw}/{ll}", got, exp)


def test_orpo_w_zero_closed_form(flce):
    B, T, H, V, beta = 3, 20, 64, 512, 0.7
    h, W, t = _inputs(B, T, H, V, seed=52, prompt_max=5, pad_max=5)
    say("orpo W = 0")
    loss, seq, gh, gw = flce.orpo_fwd_bwd(h.cuda(), torch.zeros_like(W).cuda(), t.cuda(), B, T,
                                          beta, 2)
    torch.cuda.synchronize()
    assert rel(float(loss), math.log(V) + beta * math.log(2.0)) < 1e-6
    assert torch.allclose(seq.cpu(), torch.full((2 * B,), -math.log(V)), rtol=1e-6)
    assert torch.count_nonzero(gh).item() == 0
    _, _, gw0, _ = oracle.orpo(to_float64(h), np.zeros((V, H)), t.numpy().astype(np.int64), B, T,
                               beta)
    assert rel_fro(f64(gw), gw0) <= GRAD_RTOL


def test_orpo_beta_zero_is_head_on_chosen_rows(flce):
    """beta = 0 leaves the head's mean cross entropy over the counted chosen
    rows: the same loss and grad_W as flce_fwd_bwd on that sub-batch, and
    grad_h zero outside it."""
    B, T, H, V = 4, 64, 256, 2048
    h, W, t = _inputs(B, T, H, V, seed=53, prompt_max=20, pad_max=10)
    hd, Wd, td = h.cuda(), W.cuda(), t.cuda()
    say("orpo beta = 0 vs the head")
    loss, _, gh, gw = flce.orpo_fwd_bwd(hd, Wd, td, B, T, 0.0, 2)
    rows = torch.nonzero(td[: B * T] >= 0)[:, 0]
    l2, gh2, gw2 = flce.fwd_bwd(hd[rows].contiguous(), Wd, td[rows].contiguous(), 256)
    torch.cuda.synchronize()
    assert rel(float(loss), float(l2)) < 1e-5
    assert rel_fro(f64(gw), f64(gw2)) < 5e-3
    assert rel_fro(f64(gh[rows]), f64(gh2)) < 5e-3
    mask = torch.ones(2 * B * T, dtype=torch.bool, device="cuda")
    mask[rows] = False
    assert torch.count_nonzero(gh[mask]).item() == 0


def test_orpo_chunking_invariance_and_determinism(flce):
    B, T, H, V = 6, 48, 128, 2048
    h, W, t = _inputs(B, T, H, V, seed=54, prompt_max=10, pad_max=10)
    hd, Wd, td = h.cuda(), W.cuda(), t.cuda()
    say("orpo chunking invariance")
    a = tuple(x.clone() for x in flce.orpo_fwd_bwd(hd, Wd, td, B, T, 0.3, 6))
    for cp in (1, 4):
        b = flce.orpo_fwd_bwd(hd, Wd, td, B, T, 0.3, cp)
        torch.cuda.synchronize()
        assert rel(float(b[0]), float(a[0])) < 1e-5
        assert torch.allclose(b[1], a[1], rtol=1e-5, atol=1e-6)
        assert rel_fro(f64(b[2]), f64(a[2])) < 2e-3
        assert rel_fro(f64(b[3]), f64(a[3])) < 2e-3
    again = flce.orpo_fwd_bwd(hd, Wd, td, B, T, 0.3, 6)
    torch.cuda.synchronize()
    for x, y in zip(a, again):
        assert torch.equal(x, y)


def test_orpo_no_hidden_allocation(flce):
    B, T, H, V, cp = 4, 256, 1024, 32000, 2
    h, W, t = _inputs(B, T, H, V, seed=55, prompt_max=64, pad_max=32, w_std=0.02)
    hd, Wd, td = h.cuda(), W.cuda(), t.cuda()
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    seq = torch.empty(2 * B, dtype=torch.float32, device="cuda")
    gh = torch.empty_like(hd)
    gw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    need = flce.orpo_workspace_bytes(B, T, H, V, cp, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    kw = dict(loss=loss, seq_logp=seq, grad_h=gh, grad_W=gw, workspace=ws)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.max_memory_allocated()
    say("orpo no hidden allocation")
    flce.orpo_fwd_bwd(hd, Wd, td, B, T, 0.1, cp, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base
    with pytest.raises(flce.FlceError):
        flce.orpo_fwd_bwd(hd, Wd, td, B, T, 0.1, cp, loss=loss, seq_logp=seq, grad_h=gh,
                          grad_W=gw, workspace=ws[: need - 16])


def test_orpo_sequence_without_counted_rows_is_nan(flce):
    B, T, H, V = 2, 8, 64, 256
    h, W, t = _inputs(B, T, H, V, seed=56, prompt_max=0, pad_max=0)
    t[3 * T: 4 * T] = IGNORE  # the rejected sequence of pair 1
    say("orpo empty sequence")
    loss, seq, _, _ = flce.orpo_fwd_bwd(h.cuda(), W.cuda(), t.cuda(), B, T, 0.1, 1)
    torch.cuda.synchronize()
    assert math.isnan(float(loss)) and math.isnan(float(seq[3]))
    assert not math.isnan(float(seq[0]))


def test_orpo_out_of_range_target_is_nan_not_a_fault(flce):
    B, T, H, V = 2, 8, 64, 256
    h, W, t = _inputs(B, T, H, V, seed=59, prompt_max=0, pad_max=0)
    t[5] = V  # a chosen row of pair 0
    say("orpo out-of-range target")
    loss, seq, gh, gw = flce.orpo_fwd_bwd(h.cuda(), W.cuda(), t.cuda(), B, T, 0.1, 1)
    torch.cuda.synchronize()
    assert math.isnan(float(loss)) and math.isnan(float(seq[0]))
    assert not math.isnan(float(seq[1]))


def test_orpo_llama2_like_head(flce):
    """A Llama-2-7B-like vocabulary (V = 32000) at H = 1024: 2 pairs of 512
    tokens, one pair per chunk, against the oracle element by element."""
    B, T, H, V = 2, 512, 1024, 32000
    h, W, t = _inputs(B, T, H, V, seed=57, prompt_max=128, pad_max=64, w_std=0.02)
    say("orpo V=32000 H=1024 2 x 512 tokens")
    got = flce.orpo_fwd_bwd(h.cuda(), W.cuda(), t.cuda(), B, T, 0.1, 1)
    torch.cuda.synchronize()
    _check("orpo llama2-like", got, _oracle(h, W, t, B, T, 0.1))


def test_orpo_full_size_sampled(flce):
    """The benchmark's preference batch (Llama-3-8B head, 4 pairs of 1024
    tokens, prompts and padding ignored, beta 0.1) in the benchmark's launch
    configuration (2 pairs a chunk): loss, every sequence's mean
    log-probability and sampled rows of grad_h and grad_W against the
    oracle's stored values, plus properties that hold at any size (columns
    of grad_W sum to zero; ignored rows have zero grad_h)."""
    import os
    from synth import config_by_name, make_inputs
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                     "orpo_llama3_8b_head_sampled.npz")
    if not os.path.exists(p):
        pytest.fail(f"missing {p}: run tests/golden/make_golden.py orpo")
    gold = np.load(p, allow_pickle=False)
    B, T, beta = int(gold["pairs"]), int(gold["seq_len"]), float(gold["beta"])
    say("orpo full size: generating inputs")
    inp = make_inputs(config_by_name(str(gold["config"])), seed=0)
    t = mask_preference_rows(inp.t, B, T, seed=0, prompt_max=int(gold["prompt_max"]),
                             pad_max=int(gold["pad_max"]))
    h, W, td = inp.h.cuda(), inp.W.cuda(), t.cuda()
    del inp
    say(f"orpo full size: pairs={B} seq_len={T} chunk_pairs=2")
    loss, seq, gh, gw = flce.orpo_fwd_bwd(h, W, td, B, T, beta, 2)
    torch.cuda.synchronize()
    rows = torch.from_numpy(gold["rows"]).cuda()
    vrows = torch.from_numpy(gold["vocab_rows"]).cuda()
    el = rel(float(loss), float(gold["loss"]))
    es = float(np.max(np.abs(f64(seq) - gold["seq_logp"]) / np.abs(gold["seq_logp"])))
    eh = rel_fro(f64(gh[rows]), gold["grad_h_rows"])
    ew = rel_fro(f64(gw[vrows]), gold["grad_W_rows"])
    colsum = gw.double().sum(dim=0).abs().max().item()
    scale = gw.double().abs().sum(dim=0).max().item()
    ignored = torch.count_nonzero(gh[td < 0]).item()
    say(f"  loss {float(loss):.7f} vs {float(gold['loss']):.7f} rel {el:.2e}; seq_logp "
        f"{es:.2e}; grad_h rows {eh:.2e}; grad_W rows {ew:.2e}; |sum_j grad_W| {colsum:.2e} "
        f"(sum |.| {scale:.2e}); nonzero ignored grad_h {ignored}")
    assert el <= LOSS_RTOL and es <= 1e-4 and eh <= GRAD_RTOL and ew <= GRAD_RTOL
    assert colsum <= 1e-3 * scale
    assert ignored == 0
