"""GPU parity of the training-side entry points (the steps on either side of
the fused call): gradient accumulation over micro-batches, scaling of the
precomputed gradients by the loss's upstream gradient, and the autograd
wrapper built from them.  References are the fp64 oracle on the same stored
inputs; the scaling kernel is compared bit for bit with the same fp32
product rounded on the CPU.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import make_random, to_float64
from parity_util import GRAD_RTOL, LOSS_RTOL, f64, rel, rel_fro, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def flce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_06_amd as m
    m.load()
    return m


def _oracle(inp):
    return oracle.flce(to_float64(inp.h), to_float64(inp.W), inp.t.numpy().astype(np.int64))


# shapes on both layouts of the logits: exponentiated bf16 (H % 64 == 0,
# V % 8 == 0) and fp32 (everything else), plus the fp32-input path
SHAPES = [(300, 128, 1000, 128, "bf16"), (77, 136, 523, 32, "bf16"), (50, 64, 200, 16, "f32")]


@pytest.mark.parametrize("N,H,V,chunk,dtype", SHAPES)
def test_accumulate_over_micro_batches(flce, N, H, V, chunk, dtype):
    """grad_W (+)= over two micro-batches sharing W, starting from a
    non-zero buffer: equals start + the sum of the oracle's grad_W."""
    a = make_random(N, H, V, dtype=dtype, seed=11, w_std=0.3)
    b = make_random(N, H, V, dtype=dtype, seed=12, w_std=0.3)
    b = type(b)(h=b.h, W=a.W, t=b.t, dtype=b.dtype)  # same weight, other tokens and targets
    ha, W, ta = to_device(a)
    hb, _, tb = to_device(b)
    g = torch.Generator().manual_seed(5)
    start = torch.randn(V, H, generator=g, dtype=torch.float32) * 1e-4
    gw = start.cuda()
    say(f"flce_fwd_bwd_accumulate N={N} H={H} V={V} chunk={chunk} {dtype}")
    la, gha, _ = flce.fwd_bwd(ha, W, ta, chunk, grad_W=gw, accumulate=True)
    la = float(la)
    lb, ghb, _ = flce.fwd_bwd(hb, W, tb, chunk, grad_W=gw, accumulate=True)
    torch.cuda.synchronize()
    ea, eb = _oracle(a), _oracle(b)
    exp_w = start.double().numpy() + ea[2] + eb[2]
    ew = rel_fro(f64(gw) - start.double().numpy(), ea[2] + eb[2])
    say(f"  loss {la:.6f}/{float(lb):.6f}; accumulated grad_W rel_fro {ew:.2e}")
    assert rel(la, ea[0]) <= LOSS_RTOL and rel(float(lb), eb[0]) <= LOSS_RTOL
    assert rel_fro(f64(ghb), eb[1]) <= GRAD_RTOL      # grad_h is overwritten, not summed
    assert ew <= GRAD_RTOL
    assert rel_fro(f64(gw), exp_w) <= GRAD_RTOL


@pytest.mark.parametrize("nh,nw", [(1003, 1001), (8, 4), (0, 37), (4096 * 17 + 5, 0)])
def test_scale_grads_bitwise(flce, nh, nw):
    g = torch.Generator().manual_seed(nh + nw)
    gh = (torch.randn(max(nh, 1), generator=g) * 3).to(torch.bfloat16)[:nh].contiguous()
    gw = (torch.randn(max(nw, 1), generator=g) * 3)[:nw].contiguous()
    s = torch.tensor([0.3], dtype=torch.float32)
    exp_h = (gh.float() * s).to(torch.bfloat16)   # fp32 product, round to nearest even
    exp_w = gw * s
    dh, dw = gh.cuda(), gw.cuda()
    say(f"flce_scale_grads n_h={nh} n_W={nw}")
    flce.scale_grads(dh if nh else None, dw if nw else None, s.cuda())
    torch.cuda.synchronize()
    assert torch.equal(dh.cpu().view(torch.int16), exp_h.view(torch.int16))
    assert torch.equal(dw.cpu(), exp_w)


@pytest.mark.parametrize("N,H,V,chunk,dtype", SHAPES[:2])
def test_autograd_backward(flce, N, H, V, chunk, dtype):
    """(loss * c).backward() gives c times the oracle's gradients; the loss
    value is the oracle's."""
    inp = make_random(N, H, V, dtype=dtype, seed=21, w_std=0.3)
    h0, W0, t = to_device(inp)
    h = h0.clone().requires_grad_(True)
    W = W0.clone().requires_grad_(True)
    c = 0.25  # as when a loss is divided by 4 accumulation steps
    say(f"autograd N={N} H={H} V={V} chunk={chunk} {dtype}")
    loss = flce.linear_cross_entropy(h, W, t, chunk)
    (loss * c).backward()
    torch.cuda.synchronize()
    l0, gh0, gw0 = _oracle(inp)
    eh, ew = rel_fro(f64(h.grad), c * gh0), rel_fro(f64(W.grad), c * gw0)
    lv = float(loss.detach())
    say(f"  loss rel {rel(lv, l0):.2e}; h.grad rel_fro {eh:.2e}; W.grad rel_fro {ew:.2e}")
    assert h.grad.dtype == h.dtype and W.grad.dtype == W.dtype
    assert rel(lv, l0) <= LOSS_RTOL
    assert eh <= GRAD_RTOL and ew <= GRAD_RTOL


def test_autograd_only_weight_grad(flce):
    """A frozen input (h without requires_grad) gets no gradient; W does."""
    inp = make_random(64, 64, 256, dtype="bf16", seed=31, w_std=0.3)
    h, W0, t = to_device(inp)
    W = W0.clone().requires_grad_(True)
    say("autograd, W only")
    loss = flce.linear_cross_entropy(h, W, t, 32)
    loss.backward()
    torch.cuda.synchronize()
    _, _, gw0 = _oracle(inp)
    assert h.grad is None
    assert rel_fro(f64(W.grad), gw0) <= GRAD_RTOL
