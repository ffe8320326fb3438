"""Pins of the oracle's RMSNorm-in-front-of-the-head function, flce_rmsnorm.

Facts that do not come from the oracle's own code:
* torch on the CPU in fp64 (its own RMS normalisation written with torch ops,
  cross_entropy and autograd) gives the same loss and gradients;
* central finite differences of the loss against every entry of x and gamma;
* gamma = 0 makes h = 0: loss = ln V, grad_x = 0, and grad_gamma closed form;
* with eps = 0, scaling a row of x by c > 0 leaves h and the loss unchanged
  and divides that row of grad_x by c;
* with eps = 0, every row of grad_x is orthogonal to that row of x
  (sum_k grad_x_ik x_ik = 0: the loss does not change along x_i);
* gamma = 1, eps = 0 on rows of mean square 1 reduces to the plain head.
``test_rmsnorm_mutants_are_caught`` plants plausible mistakes in copies and
checks that a pin rejects each.
"""

import math

import numpy as np
import pytest
import torch

from oracle import flce, flce_rmsnorm, rmsnorm


def _rand(N, H, V, seed=0, x_std=1.5, w_std=0.5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H)) * x_std
    g = 1.0 + 0.3 * rng.standard_normal(H)
    W = rng.standard_normal((V, H)) * w_std
    t = rng.integers(0, V, N)
    return x, g, W, t


def _close(a, b, rtol=1e-10, atol=1e-13):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.allclose(a, b, rtol=rtol, atol=atol), float(np.max(np.abs(a - b)))


def pin_torch(impl):
    x, g, W, t = _rand(6, 8, 11, seed=1)
    eps = 1e-6
    loss, gx, gg, gw = impl(x, g, eps, W, t)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    h = xt * torch.rsqrt(xt.pow(2).mean(dim=1, keepdim=True) + eps) * gt
    lt = torch.nn.functional.cross_entropy(h @ Wt.T, torch.tensor(t))
    lt.backward()
    assert abs(loss - lt.item()) <= 1e-12 * max(1.0, abs(lt.item()))
    _close(gx, xt.grad.numpy())
    _close(gg, gt.grad.numpy())
    _close(gw, Wt.grad.numpy())


def pin_finite_differences(impl):
    x, g, W, t = _rand(3, 4, 5, seed=2)
    eps = 1e-3
    _, gx, gg, _ = impl(x, g, eps, W, t)
    d = 1e-6
    for (i, k) in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[i, k] += d
        xm[i, k] -= d
        fd = (impl(xp, g, eps, W, t)[0] - impl(xm, g, eps, W, t)[0]) / (2 * d)
        assert abs(fd - gx[i, k]) <= 1e-7 * max(1.0, abs(fd)), (i, k, fd, gx[i, k])
    for k in range(g.shape[0]):
        gp, gm = g.copy(), g.copy()
        gp[k] += d
        gm[k] -= d
        fd = (impl(x, gp, eps, W, t)[0] - impl(x, gm, eps, W, t)[0]) / (2 * d)
        assert abs(fd - gg[k]) <= 1e-7 * max(1.0, abs(fd)), (k, fd, gg[k])


def pin_gamma_zero(impl):
    x, g, W, t = _rand(7, 6, 9, seed=3)
    N, V = x.shape[0], W.shape[0]
    loss, gx, gg, gw = impl(x, np.zeros_like(g), 1e-6, W, t)
    assert abs(loss - math.log(V)) <= 1e-12
    assert np.abs(gx).max() == 0.0
    # h = 0: grad_h = (mean_j W_j - W_{t_i}) / N, grad_gamma = sum_i grad_h_i * x_i r_i
    r = 1.0 / np.sqrt((x * x).mean(axis=1) + 1e-6)
    gh = (W.mean(axis=0)[None, :] - W[t]) / N
    _close(gg, (gh * x * r[:, None]).sum(axis=0))
    assert np.abs(gw).max() == 0.0


def pin_row_scale_invariance(impl):
    x, g, W, t = _rand(5, 6, 7, seed=4)
    l0, gx0, gg0, _ = impl(x, g, 0.0, W, t)
    c = np.array([1.0, 3.0, 0.25, 7.0, 0.5])
    l1, gx1, gg1, _ = impl(x * c[:, None], g, 0.0, W, t)
    assert abs(l0 - l1) <= 1e-12 * max(1.0, abs(l0))
    _close(gx1 * c[:, None], gx0)
    _close(gg1, gg0)
    # the loss does not change along x_i: sum_k grad_x_ik x_ik = 0
    assert np.abs((gx0 * x).sum(axis=1)).max() <= 1e-12


def pin_reduces_to_head(impl):
    """gamma = 1, eps = 0 on rows of mean square 1: h = x exactly."""
    x, g, W, t = _rand(4, 8, 6, seed=5)
    x = x / np.sqrt((x * x).mean(axis=1, keepdims=True))
    loss, _, _, gw = impl(x, np.ones_like(g), 0.0, W, t)
    l0, _, gw0 = flce(x, W, t)
    assert abs(loss - l0) <= 1e-12 * max(1.0, abs(l0))
    _close(gw, gw0)


PINS = [pin_torch, pin_finite_differences, pin_gamma_zero, pin_row_scale_invariance,
        pin_reduces_to_head]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_rmsnorm_oracle_pins(pin):
    pin(flce_rmsnorm)


def test_rmsnorm_definition():
    x, g, _, _ = _rand(3, 5, 2, seed=6)
    h, r = rmsnorm(x, g, 1e-6)
    for i in range(3):
        ms = sum(v * v for v in x[i]) / 5
        for k in range(5):
            assert abs(h[i, k] - x[i, k] / math.sqrt(ms + 1e-6) * g[k]) <= 1e-14
        assert abs(r[i] - 1.0 / math.sqrt(ms + 1e-6)) <= 1e-14


# planted mistakes ----------------------------------------------------------

def _mut_no_correction(x, g, eps, W, t):
    # grad_x without the term through r (treats r as a constant)
    loss, gx, gg, gw = flce_rmsnorm(x, g, eps, W, t)
    h, r = rmsnorm(x, g, eps)
    _, gh, _ = flce(h, W, t)
    return loss, r[:, None] * g[None, :] * gh, gg, gw


def _mut_eps_outside(x, g, eps, W, t):
    # eps added to the root instead of the mean square
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / (np.sqrt((x * x).mean(axis=1)) + eps)
    h = x * r[:, None] * g[None, :]
    loss, gh, gw = flce(h, W, t)
    H = x.shape[1]
    dot = (gh * g[None, :] * x).sum(axis=1)
    gx = r[:, None] * g[None, :] * gh - x * (r ** 3 / H * dot)[:, None]
    return loss, gx, (gh * x * r[:, None]).sum(axis=0), gw


def _mut_gamma_grad_without_r(x, g, eps, W, t):
    loss, gx, gg, gw = flce_rmsnorm(x, g, eps, W, t)
    h, r = rmsnorm(x, g, eps)
    _, gh, _ = flce(h, W, t)
    return loss, gx, (gh * x).sum(axis=0), gw


def _mut_sum_not_mean(x, g, eps, W, t):
    # sum of squares instead of their mean (the chain rule redone for it)
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt((x * x).sum(axis=1) + eps)
    h = x * r[:, None] * g[None, :]
    loss, gh, gw = flce(h, W, t)
    dot = (gh * g[None, :] * x).sum(axis=1)
    gx = r[:, None] * g[None, :] * gh - x * (r ** 3 * dot)[:, None]
    return loss, gx, (gh * x * r[:, None]).sum(axis=0), gw


MUTANTS = [_mut_no_correction, _mut_eps_outside, _mut_gamma_grad_without_r, _mut_sum_not_mean]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_rmsnorm_mutants_are_caught(mutant):
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin rejects {mutant.__name__}"
