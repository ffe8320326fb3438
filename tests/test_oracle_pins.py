"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each pin is a function ``pin_*(impl)`` that raises AssertionError when the
implementation ``impl(h, W, t) -> (loss, grad_h, grad_W)`` breaks a fact the
mathematics of the loss head fixes:

* closed forms: W = 0 and h = 0 (uniform softmax, loss = ln V), and
  two-valued logits from a permutation-matrix weight;
* central finite differences of the loss against every gradient entry;
* an independent library implementation (torch's cross_entropy + autograd
  on the CPU, fp64);
* invariants: zero row sums of dloss/dZ (so the columns of grad_W sum to 0),
  shift invariance of W's rows, token and vocabulary permutations;
* brute force (pure-Python loops) and chunked == unchunked.

``test_mutants_are_caught`` plants plausible mistakes in copies of the oracle
(on the CPU) and checks that at least one pin rejects each of them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import flce, flce_brute, flce_chunked, flce_sampled, flce_vocab_chunked

RTOL = 1e-11


def _rand(N, H, V, seed=0, h_std=1.0, w_std=0.5):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H)) * h_std
    W = rng.standard_normal((V, H)) * w_std
    t = rng.integers(0, V, N)
    return h, W, t


def _close(a, b, rtol=RTOL, atol=1e-14):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1.0)
    assert err <= rtol * scale + atol, f"max abs err {err:.3e} (scale {scale:.3e})"


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_w_zero(impl):
    """W = 0: every logit is 0, softmax is uniform, loss = ln V,
    grad_h = 0, grad_W[j] = (1/N)((1/V) sum_i h_i - sum_{i: t_i = j} h_i)."""
    N, H, V = 7, 5, 6
    h, _, t = _rand(N, H, V, seed=1)
    W = np.zeros((V, H))
    loss, gh, gw = impl(h, W, t)
    assert abs(loss - math.log(V)) <= 1e-14, loss
    _close(gh, np.zeros((N, H)))
    exp_gw = np.tile(h.sum(axis=0) / V, (V, 1))
    for i in range(N):
        exp_gw[t[i]] -= h[i]
    _close(gw, exp_gw / N)


def pin_h_zero(impl):
    """h = 0: loss = ln V, grad_W = 0,
    grad_h[i] = (1/N)((1/V) sum_j W_j - W_{t_i})."""
    N, H, V = 5, 4, 9
    _, W, t = _rand(N, H, V, seed=2)
    h = np.zeros((N, H))
    loss, gh, gw = impl(h, W, t)
    assert abs(loss - math.log(V)) <= 1e-14, loss
    _close(gw, np.zeros((V, H)))
    exp_gh = (W.mean(axis=0)[None, :] - W[t]) / N
    _close(gh, exp_gh)


def pin_two_valued(impl):
    """W is a permutation matrix (row j = e_{pi(j)}), h_i = a e_{pi(t_i)}:
    Z_ij = a [j = t_i], so loss = ln(e^a + V - 1) - a for every row and
    dloss/dZ is known in closed form; grad_h[i, pi(j)] = G_ij and
    grad_W[j, pi(t_i)] accumulates a G_ij."""
    N, V, H = 6, 5, 7
    a = 4.0
    rng = np.random.default_rng(3)
    pi = rng.permutation(H)[:V]
    t = rng.integers(0, V, N)
    W = np.zeros((V, H))
    W[np.arange(V), pi] = 1.0
    h = np.zeros((N, H))
    h[np.arange(N), pi[t]] = a
    loss, gh, gw = impl(h, W, t)
    denom = math.exp(a) + V - 1
    assert abs(loss - (math.log(denom) - a)) <= 1e-14
    G = np.full((N, V), 1.0 / denom)
    G[np.arange(N), t] = math.exp(a) / denom - 1.0
    G /= N
    exp_gh = np.zeros((N, H))
    exp_gh[:, pi] = G
    exp_gw = np.zeros((V, H))
    for i in range(N):
        exp_gw[:, pi[t[i]]] += a * G[i]
    _close(gh, exp_gh)
    _close(gw, exp_gw)


def pin_torch_autograd(impl):
    """torch's own cross_entropy (mean reduction) and autograd, fp64 CPU."""
    for (N, H, V, seed) in [(9, 6, 11, 4), (1, 3, 2, 5), (16, 8, 33, 6)]:
        h, W, t = _rand(N, H, V, seed=seed)
        th = torch.tensor(h, requires_grad=True)
        tW = torch.tensor(W, requires_grad=True)
        tl = torch.nn.functional.cross_entropy(th @ tW.T, torch.tensor(t))
        tl.backward()
        loss, gh, gw = impl(h, W, t)
        assert abs(loss - tl.item()) <= 1e-12 * max(1.0, abs(tl.item()))
        _close(gh, th.grad.numpy())
        _close(gw, tW.grad.numpy())


def pin_finite_differences(impl):
    """Central differences of the loss against every entry of both grads."""
    N, H, V = 3, 4, 5
    h, W, t = _rand(N, H, V, seed=7)
    _, gh, gw = impl(h, W, t)
    eps = 1e-5
    for arr, grad in ((h, gh), (W, gw)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = impl(h, W, t)[0]
            arr[idx] = old - eps
            lm = impl(h, W, t)[0]
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - grad)) / max(np.max(np.abs(grad)), 1e-300)
        assert err < 1e-7, f"finite-difference mismatch {err:.3e}"


def pin_row_sums(impl):
    """softmax rows sum to 1, so G rows sum to 0 and sum_j grad_W[j,:] = 0."""
    h, W, t = _rand(12, 5, 17, seed=8)
    _, _, gw = impl(h, W, t)
    scale = np.abs(gw).max()
    assert np.max(np.abs(gw.sum(axis=0))) <= 1e-13 * max(scale, 1.0)


def pin_shift_invariance(impl):
    """Adding one vector c to every row of W adds h_i.c to every logit of
    row i: loss and G are unchanged, so grad_h and grad_W are too."""
    h, W, t = _rand(8, 6, 10, seed=9)
    c = np.random.default_rng(10).standard_normal(6) * 3.0
    l0, gh0, gw0 = impl(h, W, t)
    l1, gh1, gw1 = impl(h, W + c[None, :], t)
    assert abs(l0 - l1) <= 1e-12 * max(1.0, abs(l0))
    _close(gh1, gh0, rtol=1e-10)
    _close(gw1, gw0, rtol=1e-10)


def pin_permutations(impl):
    """Permuting tokens permutes grad_h rows; permuting vocabulary rows of W
    (and relabelling t) permutes grad_W rows; the loss is unchanged."""
    N, H, V = 10, 4, 7
    h, W, t = _rand(N, H, V, seed=11)
    l0, gh0, gw0 = impl(h, W, t)
    rng = np.random.default_rng(12)
    p = rng.permutation(N)
    l1, gh1, gw1 = impl(h[p], W, t[p])
    assert abs(l0 - l1) <= 1e-13 * max(1, abs(l0))
    _close(gh1, gh0[p])
    _close(gw1, gw0)
    q = rng.permutation(V)           # new row r holds old row q[r]
    inv = np.argsort(q)              # old label j is now row inv[j]
    l2, gh2, gw2 = impl(h, W[q], inv[t])
    assert abs(l0 - l2) <= 1e-13 * max(1, abs(l0))
    _close(gh2, gh0)
    _close(gw2, gw0[q])


def pin_brute_force(impl):
    """Pure-Python loops over the definition, no numpy arithmetic."""
    for (N, H, V, seed) in [(4, 3, 6, 13), (2, 5, 3, 14), (8, 6, 10, 15)]:
        h, W, t = _rand(N, H, V, seed=seed)
        lb, ghb, gwb = flce_brute(h, W, t)
        loss, gh, gw = impl(h, W, t)
        assert abs(loss - lb) <= 1e-13 * max(1, abs(lb))
        _close(gh, ghb)
        _close(gw, gwb)


PINS = [
    pin_w_zero,
    pin_h_zero,
    pin_two_valued,
    pin_torch_autograd,
    pin_finite_differences,
    pin_row_sums,
    pin_shift_invariance,
    pin_permutations,
    pin_brute_force,
]


def _chunked(c):
    return lambda h, W, t: flce_chunked(h, W, t, c)


def _vocab_chunked(c):
    return lambda h, W, t: flce_vocab_chunked(h, W, t, c)


IMPLS = {
    "plain": flce,
    "chunk1": _chunked(1),
    "chunk2": _chunked(2),
    "chunk3": _chunked(3),
    "chunk_big": _chunked(1000),
    "vchunk1": _vocab_chunked(1),
    "vchunk2": _vocab_chunked(2),
    "vchunk3": _vocab_chunked(3),
    "vchunk_big": _vocab_chunked(1000),
    "sampled_all_rows": None,  # filled below
}


def _sampled_impl(h, W, t):
    N, V = h.shape[0], W.shape[0]
    r = flce_sampled(h, W, t, rows=np.arange(N), vocab_rows=np.arange(V), chunk=2)
    return r["loss"], r["grad_h_rows"], r["grad_W_rows"]


IMPLS["sampled_all_rows"] = _sampled_impl


@pytest.mark.parametrize("impl_name", list(IMPLS))
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin, impl_name):
    pin(IMPLS[impl_name])


def test_brute_force_itself_matches_torch():
    """The brute-force loops are pinned to torch too (not only to numpy)."""
    pin_torch_autograd(flce_brute)


def test_chunked_equals_unchunked_tiny():
    h, W, t = _rand(7, 5, 9, seed=20)
    l0, gh0, gw0 = flce(h, W, t)
    for c in (1, 2, 6, 7, 50):
        l1, gh1, gw1 = flce_chunked(h, W, t, c)
        assert abs(l0 - l1) <= 1e-14 * max(1, abs(l0))
        _close(gh1, gh0, rtol=1e-14)
        _close(gw1, gw0, rtol=1e-14)


def test_vocab_chunked_equals_unchunked():
    """Vocabulary chunks (running max/sum merge, then the gradients chunk by
    chunk) reach the unchunked result, including chunks whose maximum is
    below an earlier chunk's and logits large enough that exp overflows
    without the shift."""
    for (N, H, V, seed, w_std) in [(7, 5, 9, 22, 0.5), (5, 16, 40, 23, 20.0)]:
        h, W, t = _rand(N, H, V, seed=seed, w_std=w_std)
        l0, gh0, gw0 = flce(h, W, t)
        for c in (1, 2, 4, V - 1, V, 3 * V):
            l1, gh1, gw1 = flce_vocab_chunked(h, W, t, c)
            assert np.isfinite(l1)
            assert abs(l0 - l1) <= 1e-12 * max(1, abs(l0))
            _close(gh1, gh0, rtol=1e-12)
            _close(gw1, gw0, rtol=1e-12)


def test_large_logits_stay_finite():
    """Page 3's own example draws both h and W from N(0, 1): logits of
    standard deviation sqrt(H).  The shifted log-sum-exp must stay finite and
    agree with scipy's logsumexp."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(21)
    N, H, V = 4, 4096, 300
    h = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H))
    t = rng.integers(0, V, N)
    loss, gh, gw = flce(h, W, t)
    assert np.isfinite(loss) and np.isfinite(gh).all() and np.isfinite(gw).all()
    Z = h @ W.T
    ref = np.mean(logsumexp(Z, axis=1) - Z[np.arange(N), t])
    assert abs(loss - ref) <= 1e-12 * abs(ref)


def test_invalid_inputs_rejected():
    h, W, t = _rand(3, 2, 4)
    with pytest.raises(ValueError):
        flce(h, W, np.array([0, 4, 1]))
    with pytest.raises(ValueError):
        flce(h, W, np.array([0, -1, 1]))
    with pytest.raises(ValueError):
        flce(np.zeros((0, 2)), W, np.zeros(0, dtype=np.int64))
    with pytest.raises(ValueError):
        flce_chunked(h, W, t, 0)


def test_single_class_vocab():
    """V = 1: the only class always has probability 1, loss 0, grads 0."""
    h, W, t = _rand(5, 3, 1, seed=22)
    loss, gh, gw = flce(h, W, t)
    assert loss == 0.0
    assert np.all(gh == 0) and np.all(gw == 0)


# --------------------------------------------------------------------------
# planted mistakes: each must be rejected by at least one pin
# --------------------------------------------------------------------------

def _mut_sign(h, W, t):
    l, gh, gw = flce(h, W, t)
    return l, -gh, -gw


def _mut_drop_onehot(h, W, t):
    N = h.shape[0]
    Z = h @ W.T
    P = np.exp(Z - oracle.logsumexp_rows(Z)[:, None]) / N
    return float(oracle.row_losses(Z, t).mean()), P @ W, P.T @ h


def _mut_wrong_denominator(h, W, t):
    N = h.shape[0]
    Z = h @ W.T
    G = oracle.dlogits(Z, t, N + 1)
    return float(oracle.row_losses(Z, t).sum() / N), G @ W, G.T @ h


def _mut_local_chunk_n(h, W, t):
    # the classic chunking slip: divide each chunk by its own size
    N = h.shape[0]
    c = 2
    loss = 0.0
    gh = np.empty_like(h)
    gw = np.zeros_like(W)
    for r0 in range(0, N, c):
        r1 = min(N, r0 + c)
        Z = h[r0:r1] @ W.T
        loss += oracle.row_losses(Z, t[r0:r1]).sum() / N
        G = oracle.dlogits(Z, t[r0:r1], r1 - r0)
        gh[r0:r1] = G @ W
        gw += G.T @ h[r0:r1]
    return loss, gh, gw


def _mut_lse_without_max(h, W, t):
    Z = h @ W.T
    m = Z.max(axis=1)
    lse = np.log(np.exp(Z - m[:, None]).sum(axis=1))  # forgot "+ m"
    N = h.shape[0]
    loss = float(np.mean(lse - Z[np.arange(N), t]))
    P = np.exp(Z - (lse + m)[:, None])
    P[np.arange(N), t] -= 1
    G = P / N
    return loss, G @ W, G.T @ h


def _mut_target_shift(h, W, t):
    V = W.shape[0]
    l, _, _ = flce(h, W, t)
    _, gh, gw = flce(h, W, (t + 1) % V)
    return l, gh, gw


def _mut_softmax_wrong_axis(h, W, t):
    N = h.shape[0]
    Z = h @ W.T
    m = Z.max(axis=0)
    P = np.exp(Z - m[None, :])
    P /= P.sum(axis=0, keepdims=True)
    loss = float(oracle.row_losses(Z, t).mean())
    P[np.arange(N), t] -= 1
    G = P / N
    return loss, G @ W, G.T @ h


def _mut_grad_w_uses_w(h, W, t):
    # grad_W built from the wrong operand (G^T applied to W's own rows)
    l, gh, _ = flce(h, W, t)
    N = h.shape[0]
    G = oracle.dlogits(h @ W.T, t, N)
    hh = np.zeros_like(h)
    k = min(h.shape[0], W.shape[0])
    hh[:k] = W[:k]
    return l, gh, G.T @ hh


def _mut_last_chunk_only(h, W, t):
    N = h.shape[0]
    c = 3
    loss = 0.0
    gh = np.empty_like(h)
    gw = None
    for r0 in range(0, N, c):
        r1 = min(N, r0 + c)
        Z = h[r0:r1] @ W.T
        loss += oracle.row_losses(Z, t[r0:r1]).sum() / N
        G = oracle.dlogits(Z, t[r0:r1], N)
        gh[r0:r1] = G @ W
        gw = G.T @ h[r0:r1]  # overwritten instead of accumulated
    return loss, gh, gw


def _mut_vocab_merge_without_rescale(h, W, t):
    # vocabulary chunks whose sums are added without rescaling to the new max
    N, V = h.shape[0], W.shape[0]
    c = 2
    m = np.full(N, -np.inf)
    s = np.zeros(N)
    for v0 in range(0, V, c):
        Z = h @ W[v0:v0 + c].T
        mc = Z.max(axis=1)
        s = s + np.exp(Z - mc[:, None]).sum(axis=1)
        m = np.maximum(m, mc)
    lse = m + np.log(s)
    Z = h @ W.T
    loss = float((lse - Z[np.arange(N), t]).sum() / N)
    G = np.exp(Z - lse[:, None])
    G[np.arange(N), t] -= 1.0
    G /= N
    return loss, G @ W, G.T @ h


def _mut_vocab_local_lse(h, W, t):
    # each vocabulary chunk's gradient normalised by its own log-sum-exp
    N, V = h.shape[0], W.shape[0]
    c = 3
    l0, _, _ = flce(h, W, t)
    gh = np.zeros_like(h)
    gw = np.empty_like(W)
    for v0 in range(0, V, c):
        v1 = min(V, v0 + c)
        Z = h @ W[v0:v1].T
        G = np.exp(Z - oracle.logsumexp_rows(Z)[:, None])
        inside = (t >= v0) & (t < v1)
        G[np.arange(N)[inside], t[inside] - v0] -= 1.0
        G /= N
        gh += G @ W[v0:v1]
        gw[v0:v1] = G.T @ h
    return l0, gh, gw


def _mut_transposed_h(h, W, t):
    # grad_h computed with W's columns permuted (a transposed-index slip)
    l, gh, gw = flce(h, W, t)
    return l, gh[:, ::-1].copy(), gw


MUTANTS = [
    _mut_sign,
    _mut_drop_onehot,
    _mut_wrong_denominator,
    _mut_local_chunk_n,
    _mut_lse_without_max,
    _mut_target_shift,
    _mut_softmax_wrong_axis,
    _mut_grad_w_uses_w,
    _mut_last_chunk_only,
    _mut_vocab_merge_without_rescale,
    _mut_vocab_local_lse,
    _mut_transposed_h,
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_mutants_are_caught(mutant):
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin rejects {mutant.__name__}"
