"""fp64 oracle of the fused linear + cross-entropy (FLCE) loss head.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.

What is computed, and where the pages state it
-----------------------------------------------
* Page 2, "Liger-Kernel: Triton kernels that replace Hugging Face training
  ops", section "What actually gets replaced, and how the patch mechanism
  works": the fused head takes the hidden states and the LM-head weight and
  returns the loss itself; the (batch, sequence, vocab) logits are never
  materialised.
* Page 3, "Complete Guide to Liger Kernel", section
  "LigerFusedLinearCrossEntropyLoss": the call is (hidden [B*S, H],
  weight [V, H], labels [B*S]) -> scalar loss; section "LigerCrossEntropyLoss":
  the loss is the cross entropy of the logits against the labels.
* Page 1, "Liger Kernel explained", section "What does Liger Kernel actually
  fuse, and why does that cut memory?": the fused kernel produces the loss
  and its gradient together, working through the logits in chunks, so that
  chunking only changes the order of accumulation (the same page's
  measurement table asks for a numerical parity check for that reason).

The result has a plain definition, so this module writes it out:

    Z      = h W^T                                  logits        [N, V]
    lse_i  = m_i + ln sum_j exp(Z_ij - m_i),  m_i = max_j Z_ij
    loss   = (1/N) sum_i (lse_i - Z_{i, t_i})       mean over all N tokens
    G      = (softmax(Z) - onehot(t)) / N           dloss/dZ      [N, V]
    grad_h = G W                                    dloss/dh      [N, H]
    grad_W = G^T h                                  dloss/dW      [V, H]

Readings where the pages are silent (each is listed in the design notes):
the reduction is the mean over all N tokens (a bare cross-entropy call);
every target is a valid class (no ignore index); there is no bias, label
smoothing, z-loss, soft-capping or temperature; h is [N, H] and W is [V, H],
row-major.

Four implementations, all fp64:
* ``flce``          the definition above, unchunked (small inputs);
* ``flce_chunked``  the same steps over token chunks, grad_W accumulated in
                    fp64 and the 1/N taken with the global N (any size);
* ``flce_vocab_chunked``  the same result over chunks of vocabulary rows:
                    a pass of running (max, sum) statistics, then the
                    gradients chunk by chunk with the global log-sum-exp;
* ``flce_brute``    pure-Python loops (tiny inputs; pins numpy's matmul and
                    broadcasting);
``flce_rmsnorm`` puts an RMSNorm in front of the head (h = rmsnorm(x)) and
returns the gradients of its input x and weight gamma by the chain rule;
and ``flce_sampled`` for full-size checks: the loss plus chosen rows of
grad_h and grad_W, without holding an [N, V] or [V, H] array.
"""

from __future__ import annotations

import math

import numpy as np


def _check(h: np.ndarray, W: np.ndarray, t: np.ndarray) -> None:
    if h.ndim != 2 or W.ndim != 2 or t.ndim != 1:
        raise ValueError("expected h[N,H], W[V,H], t[N]")
    if h.shape[1] != W.shape[1] or h.shape[0] != t.shape[0]:
        raise ValueError("shape mismatch")
    if h.shape[0] < 1:
        raise ValueError("N must be >= 1: the mean over no tokens is undefined")
    if t.size and (t.min() < 0 or t.max() >= W.shape[0]):
        raise ValueError("targets must lie in [0, V)")


def logits(h: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Z = h W^T in fp64 (the LM-head linear layer, no bias)."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    """Per-row log-sum-exp, shifted by the row maximum so exp never overflows."""
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def row_losses(Z: np.ndarray, t: np.ndarray) -> np.ndarray:
    """Cross entropy of each row: lse_i - Z[i, t_i]."""
    return logsumexp_rows(Z) - Z[np.arange(Z.shape[0]), t]


def dlogits(Z: np.ndarray, t: np.ndarray, n_total: int) -> np.ndarray:
    """dloss/dZ for the mean loss over n_total tokens: (softmax - onehot)/N."""
    P = np.exp(Z - logsumexp_rows(Z)[:, None])
    P[np.arange(Z.shape[0]), t] -= 1.0
    return P / n_total


def flce(h: np.ndarray, W: np.ndarray, t: np.ndarray):
    """Unchunked definition: returns (loss, grad_h, grad_W) in fp64."""
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    _check(h, W, t)
    N = h.shape[0]
    Z = logits(h, W)
    loss = row_losses(Z, t).sum() / N
    G = dlogits(Z, t, N)
    return float(loss), G @ W, G.T @ h


def flce_chunked(h: np.ndarray, W: np.ndarray, t: np.ndarray, chunk: int):
    """The same result computed over token chunks of ``chunk`` rows.

    Only a [chunk, V] block of logits exists at a time.  grad_W sums the
    chunks' contributions in fp64; every chunk divides by the global N.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    _check(h, W, t)
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    N = h.shape[0]
    loss_sum = 0.0
    grad_h = np.empty_like(h)
    grad_W = np.zeros_like(W)
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        Z = logits(h[r0:r1], W)
        loss_sum += row_losses(Z, t[r0:r1]).sum()
        G = dlogits(Z, t[r0:r1], N)
        grad_h[r0:r1] = G @ W
        grad_W += G.T @ h[r0:r1]
    return float(loss_sum / N), grad_h, grad_W


def flce_vocab_chunked(h: np.ndarray, W: np.ndarray, t: np.ndarray, vchunk: int):
    """The same result computed over chunks of ``vchunk`` vocabulary rows of W
    (page 1, "Liger Kernel explained", section "What does Liger Kernel
    actually fuse, and why does that cut memory?": the logits are worked
    through in chunks over the vocabulary dimension).

    Only an [N, vchunk] block of logits exists at a time.  Pass 1 keeps, per
    row, the running maximum m and the sum s of exp(Z - m) over the chunks
    seen so far (when a chunk raises the maximum, the old sum is rescaled by
    exp(m_old - m_new)), which gives lse = m + ln s and the row loss (the
    target's logit is read in the chunk that holds it).  Pass 2 forms every
    chunk's logits again, its dloss/dZ with the global lse, adds G W_c to
    grad_h and writes G^T h into the chunk's rows of grad_W.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    _check(h, W, t)
    if vchunk < 1:
        raise ValueError("vchunk must be >= 1")
    N, V = h.shape[0], W.shape[0]
    rows = np.arange(N)
    m = np.full(N, -np.inf)
    s = np.zeros(N)
    zt = np.empty(N)
    for v0 in range(0, V, vchunk):
        v1 = min(V, v0 + vchunk)
        Z = logits(h, W[v0:v1])
        mc = Z.max(axis=1)
        m_new = np.maximum(m, mc)
        s = s * np.exp(m - m_new) + np.exp(Z - m_new[:, None]).sum(axis=1)
        m = m_new
        inside = (t >= v0) & (t < v1)
        zt[inside] = Z[rows[inside], t[inside] - v0]
    lse = m + np.log(s)
    loss = float((lse - zt).sum() / N)
    grad_h = np.zeros_like(h)
    grad_W = np.empty_like(W)
    for v0 in range(0, V, vchunk):
        v1 = min(V, v0 + vchunk)
        Z = logits(h, W[v0:v1])
        G = np.exp(Z - lse[:, None])
        inside = (t >= v0) & (t < v1)
        G[rows[inside], t[inside] - v0] -= 1.0
        G /= N
        grad_h += G @ W[v0:v1]
        grad_W[v0:v1] = G.T @ h
    return loss, grad_h, grad_W


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float):
    """RMSNorm of each row (page 3, "Complete Guide to Liger Kernel", section
    "LigerRMSNorm"; the epsilon convention page 2 warns about, section "The
    support surface is narrower than the pitch suggests", is eps added to the
    mean square): h = x / sqrt(mean_k x_k^2 + eps) * gamma.  Returns (h, r)
    with r = 1 / sqrt(mean_k x_k^2 + eps) per row."""
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    r = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    return x * r[:, None] * gamma[None, :], r


def flce_rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, W: np.ndarray, t: np.ndarray):
    """The loss head behind an RMSNorm of its input: h = rmsnorm(x), then the
    definition above.  Returns (loss, grad_x, grad_gamma, grad_W) by the chain
    rule through h = x r gamma, r = (mean x^2 + eps)^(-1/2):

        grad_x     = r (gamma * grad_h) - x r^3 / H * sum_k gamma_k grad_h_k x_k
        grad_gamma = sum_i grad_h_i * x_i r_i
    """
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    H = x.shape[1]
    h, r = rmsnorm(x, gamma, eps)
    loss, gh, gw = flce(h, W, t)
    dot = (gh * gamma[None, :] * x).sum(axis=1)
    gx = r[:, None] * gamma[None, :] * gh - x * (r ** 3 / H * dot)[:, None]
    gg = (gh * x * r[:, None]).sum(axis=0)
    return loss, gx, gg, gw


def flce_brute(h, W, t):
    """Pure-Python loops over the definition (tiny inputs only)."""
    h = [[float(x) for x in row] for row in np.asarray(h, dtype=np.float64)]
    W = [[float(x) for x in row] for row in np.asarray(W, dtype=np.float64)]
    t = [int(x) for x in np.asarray(t)]
    N, H, V = len(h), len(W[0]), len(W)
    if N < 1:
        raise ValueError("N must be >= 1")
    loss = 0.0
    G = [[0.0] * V for _ in range(N)]
    for i in range(N):
        z = [sum(h[i][k] * W[j][k] for k in range(H)) for j in range(V)]
        m = max(z)
        s = sum(math.exp(zj - m) for zj in z)
        lse = m + math.log(s)
        loss += lse - z[t[i]]
        for j in range(V):
            G[i][j] = (math.exp(z[j] - lse) - (1.0 if j == t[i] else 0.0)) / N
    grad_h = [[sum(G[i][j] * W[j][k] for j in range(V)) for k in range(H)]
              for i in range(N)]
    grad_W = [[sum(G[i][j] * h[i][k] for i in range(N)) for k in range(H)]
              for j in range(V)]
    return loss / N, np.array(grad_h), np.array(grad_W)


def flce_sampled(h, W, t, rows=(), vocab_rows=(), chunk: int = 1024):
    """Loss, per-row lse and chosen rows of grad_h / grad_W at any size.

    Streams over token chunks; holds at most a [chunk, V] logit block plus
    the requested rows.  Returns a dict with ``loss`` (float), ``lse`` [N],
    ``row_loss`` [N], ``grad_h_rows`` [len(rows), H] and ``grad_W_rows``
    [len(vocab_rows), H].
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    _check(h, W, t)
    N, H = h.shape
    rows = np.asarray(rows, dtype=np.int64)
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    lse = np.empty(N)
    row_loss = np.empty(N)
    gh = np.zeros((rows.size, H))
    gw = np.zeros((vocab_rows.size, H))
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        Z = logits(h[r0:r1], W)
        lse[r0:r1] = logsumexp_rows(Z)
        row_loss[r0:r1] = lse[r0:r1] - Z[np.arange(r1 - r0), t[r0:r1]]
        sel = np.nonzero((rows >= r0) & (rows < r1))[0]
        if sel.size:
            G = dlogits(Z[rows[sel] - r0], t[rows[sel]], N)
            gh[sel] = G @ W
        if vocab_rows.size:
            P = np.exp(Z[:, vocab_rows] - lse[r0:r1, None])
            P -= (t[r0:r1, None] == vocab_rows[None, :])
            gw += (P / N).T @ h[r0:r1]
        del Z
    return {
        "loss": float(row_loss.sum() / N),
        "lse": lse,
        "row_loss": row_loss,
        "grad_h_rows": gh,
        "grad_W_rows": gw,
    }
