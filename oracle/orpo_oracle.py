"""fp64 oracle of the odds-ratio preference (ORPO) loss over the same head.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and never by the product
path, with which it shares no code.

What the pages fix, and what is read into them
----------------------------------------------
Page 2, "Liger-Kernel: Triton kernels that replace Hugging Face training
ops", section "Installation and the one-line patch": the chunked
post-training losses are called directly with the LM-head weight, the hidden
states and the targets, and return the loss itself rather than logits; ORPO
is one of them.  The
pages give nothing more, so this module follows the published objective of
ORPO (Hong, Lee and Thorne, "ORPO: Monolithic Preference Optimization
without Reference Model", 2024), written out from its definition:

    rows        2B sequences of T tokens; sequence s holds rows [sT, (s+1)T);
                s < B is the chosen response of pair s, s >= B the rejected
                response of pair s - B
    counted     a row counts when its target is >= 0 (a negative target
                marks a prompt or padding position)
    log p_r     = Z[r, t_r] - lse_r,  Z = h W^T             (per counted row)
    l_s         = mean of log p_r over the counted rows of sequence s
    logodds_s   = l_s - ln(1 - exp(l_s))
    L_OR        = -(1/B) sum_b ln sigmoid(logodds_b - logodds_{B+b})
    L_SFT       = -(1/M) sum of log p_r over the counted chosen rows
                  (M of them in the whole batch)
    loss        = L_SFT + beta * L_OR

Gradient: with c_r = -dloss/dlog p_r (zero for rows that do not count),
dloss/dZ[r, :] = c_r (softmax(Z_r) - onehot(t_r)); grad_h = G W and
grad_W = G^T h as for the plain head.  By the chain rule, for a counted row
of pair b,

    c_r = 1/M [chosen only] + beta/B * sigmoid(-(lo_b - lo_{B+b}))
          * (+1 chosen, -1 rejected) / ((1 - exp(l_s)) n_s)

with n_s the counted rows of the row's sequence s.  A sequence with no
counted row has no mean log-probability; the result is then NaN.

A confident model needs the digits of 1 - p: the odds divide by
1 - exp(l), tiny when every token is near certain.  So when Z[r, t_r] is
the row's largest logit, log p_r is evaluated as
-log1p(sum over j != t_r of exp(Z[r, j] - Z[r, t_r])), the same number in
exact arithmetic as lse - Z_t, whose difference loses the small sum to
rounding; 1 - exp(l) is -expm1(l) and p_t - 1 in the gradient is
expm1(log p_t).  The objective has no floor: in fp64 these stay finite and
nonzero up to logit margins of several hundred.
"""

from __future__ import annotations

import math

import numpy as np


def _split(t: np.ndarray, pairs: int, seq_len: int):
    t = np.asarray(t)
    if t.shape != (2 * pairs * seq_len,):
        raise ValueError("targets must hold 2 * pairs * seq_len rows")
    return t.reshape(2 * pairs, seq_len)


def _target_logp(Z: np.ndarray, t: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """log softmax(Z)[r, t_r] for rows of Z with targets t: lse - Z_t, or,
    when Z_t is the row's largest logit, -log1p of the other classes'
    relative mass (the same value, without the cancellation)."""
    k = np.arange(Z.shape[0])
    zt = Z[k, t]
    D = Z - zt[:, None]
    D[k, t] = -np.inf
    top = D.max(axis=1) <= 0.0
    with np.errstate(over="ignore"):
        S = np.exp(D).sum(axis=1)
    return np.where(top, -np.log1p(np.where(top, S, 0.0)), zt - lse)


def token_logp(h: np.ndarray, W: np.ndarray, t: np.ndarray):
    """log softmax(h W^T)[r, t_r] for counted rows (0 elsewhere), the softmax
    P and the counted mask, all fp64."""
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t)
    V = W.shape[0]
    if np.any(t >= V):
        raise ValueError("target >= V")
    Z = h @ W.T
    m = Z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(Z - m).sum(axis=1, keepdims=True)))[:, 0]
    P = np.exp(Z - lse[:, None])
    counted = t >= 0
    logp = np.zeros(h.shape[0])
    rows = np.nonzero(counted)[0]
    logp[rows] = _target_logp(Z[rows], t[rows], lse[rows])
    return logp, P, counted


def objective(logp: np.ndarray, counted: np.ndarray, pairs: int, seq_len: int,
              beta: float):
    """The objective from per-row log-probabilities: returns (loss, c, l_seq)
    with c_r = -dloss/dlog p_r (0 for rows that do not count) and l_seq the
    mean log-probability of every sequence."""
    B, T = pairs, seq_len
    lp = logp.reshape(2 * B, T)
    cnt = counted.reshape(2 * B, T).sum(axis=1).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        l_seq = lp.sum(axis=1) / cnt                     # mean log p per sequence
        Q = -np.expm1(l_seq)                             # 1 - exp(l)
        logodds = l_seq - np.log(Q)                      # ln(P / (1 - P))
    ratio = logodds[:B] - logodds[B:]
    # -ln sigmoid(x) = ln(1 + exp(-x)), written stably
    with np.errstate(invalid="ignore"):
        l_or = float(np.mean(np.logaddexp(0.0, -ratio)))
    sig_neg = 1.0 / (1.0 + np.exp(ratio))                # sigmoid(-ratio)
    with np.errstate(divide="ignore", invalid="ignore"):
        per_seq = beta / B * np.concatenate([sig_neg, -sig_neg]) / (Q * cnt)
    M = float(counted[: B * T].sum())
    l_sft = float(-logp[: B * T].sum() / M) if M > 0 else math.nan
    loss = l_sft + beta * l_or

    # c_r = -dloss/dlog p_r
    c = np.repeat(per_seq, T)
    c[: B * T] += 1.0 / M if M > 0 else math.nan
    c = np.where(counted, c, 0.0)
    return loss, c, l_seq


def orpo(h, W, t, pairs: int, seq_len: int, beta: float):
    """ORPO loss and gradients; returns (loss, grad_h, grad_W, seq_logp)
    with seq_logp[s] the mean log-probability l_s of sequence s."""
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t)
    _split(t, pairs, seq_len)
    logp, P, counted = token_logp(h, W, t)
    loss, c, l_seq = objective(logp, counted, pairs, seq_len, beta)
    G = P
    rows = np.nonzero(counted)[0]
    G[rows, t[rows]] = np.expm1(logp[rows])  # p_t - 1, with its digits near p_t = 1
    G *= c[:, None]
    return loss, G @ W, G.T @ h, l_seq


def orpo_sampled(h, W, t, pairs: int, seq_len: int, beta: float, rows=(), vocab_rows=(),
                 chunk: int = 1024):
    """The same objective at any size: streams the logits over row chunks
    (a [chunk, V] block at a time) for every row's log-sum-exp and target
    log-probability, then forms only the requested rows of grad_h and of
    grad_W.  Returns a dict with ``loss``, ``seq_logp`` [2 pairs], ``lse``
    [N], ``grad_h_rows`` [len(rows), H] and ``grad_W_rows``
    [len(vocab_rows), H]."""
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    _split(t, pairs, seq_len)
    if np.any(t >= W.shape[0]):
        raise ValueError("target >= V")
    N = h.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    counted = t >= 0
    lse = np.empty(N)
    logp = np.zeros(N)
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        Z = h[r0:r1] @ W.T
        m = Z.max(axis=1, keepdims=True)
        lse[r0:r1] = (m + np.log(np.exp(Z - m).sum(axis=1, keepdims=True)))[:, 0]
        k = np.nonzero(counted[r0:r1])[0]
        logp[r0 + k] = _target_logp(Z[k], t[r0 + k], lse[r0 + k])
        del Z
    loss, c, l_seq = objective(logp, counted, pairs, seq_len, beta)
    gh = np.zeros((rows.size, h.shape[1]))
    if rows.size:
        Zr = h[rows] @ W.T
        Gr = np.exp(Zr - lse[rows, None])
        k = np.nonzero(counted[rows])[0]
        Gr[k, t[rows[k]]] = np.expm1(logp[rows[k]])  # p_t - 1
        gh = (Gr * c[rows, None]) @ W
    gw = np.zeros((vocab_rows.size, h.shape[1]))
    if vocab_rows.size:
        GJ = np.exp(h @ W[vocab_rows].T - lse[:, None])
        r, j = np.nonzero(t[:, None] == vocab_rows[None, :])
        GJ[r, j] = np.expm1(logp[r])  # p_t - 1 where the column is the row's target
        gw = (GJ * c[:, None]).T @ h
    return {"loss": loss, "seq_logp": l_seq, "lse": lse, "grad_h_rows": gh,
            "grad_W_rows": gw}
