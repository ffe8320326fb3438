"""Pins of the oracle's odds-ratio preference loss, ``oracle.orpo``.

Facts that do not come from the oracle's own code:
* torch on the CPU in fp64 (its own formulation: log_softmax, gather, a
  masked mean per sequence, expm1 for the odds, logsigmoid, cross_entropy
  with an ignore index for the chosen half, autograd for the gradients)
  gives the same loss, gradients and per-sequence mean log-probabilities;
* central finite differences of the loss against every entry of h and W;
* W = 0: every token has log p = -ln V, every odds ratio is 1, so
  loss = ln V + beta ln 2, grad_h = 0, and grad_W has a closed form;
* beta = 0 leaves the plain head's cross entropy over the counted chosen
  rows (the already pinned ``oracle.flce`` on that sub-batch);
* rows whose target is negative do not count: changing their hidden state
  changes nothing and their grad_h rows are zero;
* swapping the chosen and rejected halves changes the odds-ratio term by
  the mean log odds ratio (ln sigmoid(x) - ln sigmoid(-x) = x);
* two-valued logits (a token's target logit m, every other logit 0): then
  p = 1 / (1 + (V - 1) e^-m) and the odds p / (1 - p) = e^m / (V - 1)
  exactly, so the log odds are m - ln(V - 1), the odds ratio of a pair is
  the difference of its two margins, and the loss, every sequence's mean
  log-probability and every entry of grad_h have closed forms, also for a
  sequence the model is certain of (margin 40: 1 - p ~ 1e-17, far below
  what lse - Z_t resolves in fp64).
``test_orpo_mutants_are_caught`` plants plausible mistakes in copies and
checks that a pin rejects each.
"""

import math

import numpy as np
import pytest
import torch

from oracle import flce, orpo, orpo_sampled


def _rand(B, T, H, V, seed=0, h_std=1.0, w_std=0.5, ignore=()):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((2 * B * T, H)) * h_std
    W = rng.standard_normal((V, H)) * w_std
    t = rng.integers(0, V, 2 * B * T)
    for r in ignore:
        t[r] = -100
    return h, W, t


def _close(a, b, rtol=1e-10, atol=1e-13):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.allclose(a, b, rtol=rtol, atol=atol), float(np.max(np.abs(a - b)))


def _torch_ref(h, W, t, B, T, beta):
    """torch fp64: the objective in torch's own ops, gradients by autograd."""
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    tt = torch.tensor(t)
    z = ht @ Wt.T
    lsm = torch.log_softmax(z, dim=1)
    mask = tt >= 0
    tok = lsm.gather(1, tt.clamp(min=0)[:, None])[:, 0] * mask
    mean_lp = tok.view(2 * B, T).sum(dim=1) / mask.view(2 * B, T).sum(dim=1)
    lo = mean_lp - torch.log(-torch.expm1(mean_lp))
    l_or = -torch.nn.functional.logsigmoid(lo[:B] - lo[B:]).mean()
    l_sft = torch.nn.functional.cross_entropy(z[: B * T], tt[: B * T], ignore_index=-100)
    lt = l_sft + beta * l_or
    lt.backward()
    return lt.item(), ht.grad.numpy(), Wt.grad.numpy(), mean_lp.detach().numpy()


def pin_torch(impl):
    B, T, H, V, beta = 3, 4, 6, 9, 0.7
    h, W, t = _rand(B, T, H, V, seed=1, ignore=(0, 1, 13, 22))
    loss, gh, gw, seq = impl(h, W, t, B, T, beta)
    lt, gh_t, gw_t, seq_t = _torch_ref(h, W, t, B, T, beta)
    assert abs(loss - lt) <= 1e-12 * max(1.0, abs(lt))
    _close(seq, seq_t)
    _close(gh, gh_t)
    _close(gw, gw_t)


def pin_finite_differences(impl):
    B, T, H, V, beta = 2, 3, 4, 5, 1.3
    h, W, t = _rand(B, T, H, V, seed=2, ignore=(4,))
    _, gh, gw, _ = impl(h, W, t, B, T, beta)
    d = 1e-6
    for arr, grad in ((h, gh), (W, gw)):
        for idx in np.ndindex(*arr.shape):
            keep = arr[idx]
            arr[idx] = keep + d
            lp = impl(h, W, t, B, T, beta)[0]
            arr[idx] = keep - d
            lm = impl(h, W, t, B, T, beta)[0]
            arr[idx] = keep
            fd = (lp - lm) / (2 * d)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])


def pin_w_zero(impl):
    B, T, H, V, beta = 2, 5, 4, 7, 0.4
    h, _, t = _rand(B, T, H, V, seed=3, ignore=(0, 7, 12))
    W = np.zeros((V, H))
    loss, gh, gw, seq = impl(h, W, t, B, T, beta)
    assert abs(loss - (math.log(V) + beta * math.log(2.0))) <= 1e-12
    assert np.abs(gh).max() == 0.0
    _close(seq, np.full(2 * B, -math.log(V)))
    # every odds ratio is 1: sigmoid(0) = 1/2; 1 - exp(l) = 1 - 1/V
    counted = t >= 0
    n = counted.reshape(2 * B, T).sum(axis=1)
    M = counted[: B * T].sum()
    exp_gw = np.zeros((V, H))
    for r in range(2 * B * T):
        if not counted[r]:
            continue
        s = r // T
        sign = 1.0 if s < B else -1.0
        c = beta / B * 0.5 * sign / ((1.0 - 1.0 / V) * n[s])
        if s < B:
            c += 1.0 / M
        g = np.full(V, c / V)
        g[t[r]] -= c
        exp_gw += np.outer(g, h[r])
    _close(gw, exp_gw)


def pin_beta_zero_is_head_on_chosen(impl):
    B, T, H, V = 3, 4, 5, 8
    h, W, t = _rand(B, T, H, V, seed=4, ignore=(2, 5, 17))
    loss, gh, gw, _ = impl(h, W, t, B, T, 0.0)
    rows = [r for r in range(B * T) if t[r] >= 0]
    l0, gh0, gw0 = flce(h[rows], W, t[rows])
    assert abs(loss - l0) <= 1e-12 * max(1.0, abs(l0))
    _close(gw, gw0)
    exp_gh = np.zeros_like(h)
    exp_gh[rows] = gh0
    _close(gh, exp_gh)


def pin_ignored_rows(impl):
    B, T, H, V, beta = 2, 4, 5, 6, 0.9
    ign = (1, 6, 11)
    h, W, t = _rand(B, T, H, V, seed=5, ignore=ign)
    l0, gh0, gw0, _ = impl(h, W, t, B, T, beta)
    h2 = h.copy()
    h2[list(ign)] = np.random.default_rng(9).standard_normal((len(ign), H)) * 5.0
    l1, _, gw1, _ = impl(h2, W, t, B, T, beta)
    assert abs(l0 - l1) <= 1e-12 * max(1.0, abs(l0))
    _close(gw1, gw0)
    assert np.abs(gh0[list(ign)]).max() == 0.0


def pin_swap_halves(impl):
    B, T, H, V, beta = 3, 3, 4, 7, 1.0
    h, W, t = _rand(B, T, H, V, seed=6, ignore=(4,))
    loss, _, _, seq = impl(h, W, t, B, T, beta)
    n = B * T
    hs = np.concatenate([h[n:], h[:n]])
    ts = np.concatenate([t[n:], t[:n]])
    loss_s, _, _, _ = impl(hs, W, ts, B, T, beta)
    sft = lambda hh, tt: flce(hh[[r for r in range(n) if tt[r] >= 0]], W,
                              tt[[r for r in range(n) if tt[r] >= 0]])[0]
    lo = seq - np.log1p(-np.exp(seq))
    mean_ratio = float(np.mean(lo[:B] - lo[B:]))
    lhs = (loss_s - sft(hs, ts)) - (loss - sft(h, t))
    assert abs(lhs - beta * mean_ratio) <= 1e-11, (lhs, mean_ratio)


def pin_two_valued(impl):
    """Closed forms for two-valued logits.  W is the identity in the first V
    columns and a counted row of sequence s is h_r = m_s e_{t_r}, so its
    logits are m_s at the target and 0 elsewhere.  Pair b has margins
    (a_b, b_b) for its chosen and rejected sequence; with q(m) = 1 - p =
    (V-1) e^-m / (1 + (V-1) e^-m):
      log p = -log1p((V-1) e^-m),   log odds = m - ln(V-1),
      loss  = (1/M) sum over counted chosen rows of log1p((V-1) e^-a_b)
              + (beta/B) sum_b ln(1 + e^(b_b - a_b)),
      dloss/dZ[r, t_r] = -q(a_b)/M - (beta/B) sigmoid(b_b - a_b) / n_w   (chosen)
                       = +(beta/B) sigmoid(b_b - a_b) / n_l              (rejected),
    and the V - 1 other logits of the row share -(that) / (V - 1) (the row
    of G sums to zero); grad_h = G W is G itself in the first V columns."""
    V, H, T, beta = 6, 8, 4, 0.6
    margins = [(40.0, 10.0), (10.0, 40.0), (12.0, 9.5), (9.2, 9.8)]
    B = len(margins)
    rng = np.random.default_rng(11)
    t = rng.integers(0, V, 2 * B * T)
    t[[1, 6, 13, 22]] = -100
    W = np.zeros((V, H))
    W[:, :V] = np.eye(V)
    h = np.zeros((2 * B * T, H))
    m_seq = [a for a, _ in margins] + [b for _, b in margins]
    for r in range(2 * B * T):
        if t[r] >= 0:
            h[r, t[r]] = m_seq[r // T]
    loss, gh, _, seq = impl(h, W, t, B, T, beta)
    counted = t >= 0
    n = counted.reshape(2 * B, T).sum(axis=1)
    M = int(counted[: B * T].sum())
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    q = lambda m: (V - 1) * math.exp(-m) / (1.0 + (V - 1) * math.exp(-m))
    exp_loss = sum(n[b] * math.log1p((V - 1) * math.exp(-a)) for b, (a, _) in enumerate(margins))
    exp_loss = exp_loss / M + beta / B * sum(math.log1p(math.exp(bb - a)) for a, bb in margins)
    assert abs(loss - exp_loss) <= 1e-12 * exp_loss, (loss, exp_loss)
    exp_seq = np.array([-math.log1p((V - 1) * math.exp(-m)) for m in m_seq])
    assert np.allclose(seq, exp_seq, rtol=1e-12, atol=0.0), (seq, exp_seq)
    exp_gh = np.zeros_like(h)
    for r in range(2 * B * T):
        if not counted[r]:
            continue
        s = r // T
        a, bb = margins[s % B]
        if s < B:
            gt = -q(a) / M - beta / B * sig(bb - a) / n[s]
        else:
            gt = beta / B * sig(bb - a) / n[s]
        exp_gh[r, :V] = -gt / (V - 1)
        exp_gh[r, t[r]] = gt
    assert np.allclose(gh, exp_gh, rtol=1e-9, atol=0.0), float(np.max(np.abs(gh - exp_gh)))


PINS = [pin_torch, pin_finite_differences, pin_w_zero, pin_beta_zero_is_head_on_chosen,
        pin_ignored_rows, pin_swap_halves, pin_two_valued]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_orpo_oracle_pins(pin):
    pin(orpo)


def test_orpo_empty_sequence_is_nan():
    h, W, t = _rand(1, 3, 4, 5, seed=7)
    t[3:] = -100  # the rejected sequence has no counted row
    loss, gh, gw, seq = orpo(h, W, t, 1, 3, 0.1)
    assert math.isnan(loss) and math.isnan(seq[1])


@pytest.mark.parametrize("chunk", [1, 5, 7, 1000])
def test_orpo_sampled_equals_orpo(chunk):
    """The streamed form (for full-size expected values) against the pinned
    definition, for chunk sizes that do and do not divide the rows."""
    B, T, H, V, beta = 3, 5, 6, 11, 0.6
    h, W, t = _rand(B, T, H, V, seed=8, ignore=(0, 6, 7, 20, 29))
    loss, gh, gw, seq = orpo(h, W, t, B, T, beta)
    rows = np.array([0, 3, 6, 14, 29])
    vocab = np.array([0, 4, 10])
    r = orpo_sampled(h, W, t, B, T, beta, rows=rows, vocab_rows=vocab, chunk=chunk)
    assert abs(r["loss"] - loss) <= 1e-12 * abs(loss)
    _close(r["seq_logp"], seq)
    _close(r["grad_h_rows"], gh[rows])
    _close(r["grad_W_rows"], gw[vocab])


# planted mistakes ----------------------------------------------------------

def _variant(mistake):
    """A copy of the objective and its gradient with one planted mistake."""

    def impl(h, W, t, B, T, beta):
        h = np.asarray(h, dtype=np.float64)
        W = np.asarray(W, dtype=np.float64)
        t = np.asarray(t)
        Z = h @ W.T
        m = Z.max(axis=1, keepdims=True)
        lse = (m + np.log(np.exp(Z - m).sum(axis=1, keepdims=True)))[:, 0]
        P = np.exp(Z - lse[:, None])
        counted = t >= 0 if mistake != "count_ignored" else np.ones(len(t), bool)
        ar = np.arange(len(t))
        tc = np.where(t >= 0, t, 0)
        zt = Z[ar, tc]
        if mistake == "cancelling_logp":  # lse - Z_t for every row
            lp_all = zt - lse
        else:  # the other classes' mass when the target is the largest logit
            D = Z - zt[:, None]
            D[ar, tc] = -np.inf
            top = D.max(axis=1) <= 0.0
            lp_all = np.where(top, -np.log1p(np.where(top, np.exp(D).sum(axis=1), 0.0)),
                              zt - lse)
        logp = np.where(counted, lp_all, 0.0)
        cnt = counted.reshape(2 * B, T).sum(axis=1).astype(np.float64)
        norm = cnt if mistake != "sum_not_mean" else np.ones(2 * B)
        l_seq = logp.reshape(2 * B, T).sum(axis=1) / norm
        lo = l_seq - np.log(-np.expm1(l_seq)) if mistake != "odds_is_prob" else l_seq
        ratio = lo[:B] - lo[B:]
        red = np.mean if mistake != "or_sum" else np.sum
        l_or = float(red(np.logaddexp(0.0, -ratio)))
        sft_rows = slice(0, B * T) if mistake != "sft_both" else slice(0, 2 * B * T)
        M = float(counted[sft_rows].sum())
        loss = float(-logp[sft_rows].sum() / M) + beta * l_or
        sig = 1.0 / (1.0 + np.exp(ratio))
        rej = -sig if mistake != "rejected_sign" else sig
        dlo = -1.0 / np.expm1(l_seq) if mistake != "odds_is_prob" else np.ones(2 * B)
        scale = 1.0 / B if mistake != "or_sum" else 1.0
        per_seq = beta * scale * np.concatenate([sig, rej]) * dlo / norm
        c = np.repeat(per_seq, T)
        c[sft_rows] += 1.0 / M
        c = np.where(counted, c, 0.0)
        G = P.copy()
        if mistake == "cancelling_logp":
            G[ar, tc] -= np.where(counted, 1.0, 0.0)
        else:
            G[ar, tc] = np.where(counted, np.expm1(lp_all), G[ar, tc])
        G *= c[:, None]
        return loss, G @ W, G.T @ h, l_seq

    def quiet(*a):
        with np.errstate(all="ignore"):  # a planted mistake may divide by zero
            return impl(*a)

    quiet.__name__ = f"mut_{mistake}"
    return quiet


MUTANTS = ["sum_not_mean", "odds_is_prob", "or_sum", "sft_both", "rejected_sign",
           "count_ignored", "cancelling_logp"]


def test_variant_without_mistake_passes_every_pin():
    for pin in PINS:
        pin(_variant(None))


@pytest.mark.parametrize("mistake", MUTANTS)
def test_orpo_mutants_are_caught(mistake):
    caught = []
    for pin in PINS:
        try:
            pin(_variant(mistake))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin rejects {mistake}"
