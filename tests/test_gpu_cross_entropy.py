"""GPU parity of the cross entropy on given logits (flce_cross_entropy):
the mean loss, and the logits rewritten in place as dloss/dlogits, against
the fp64 oracle's row losses and logit gradient on the same stored logit
values (page 3, "Complete Guide to Liger Kernel", section
"LigerCrossEntropyLoss": [B*S, V] logits with B*S = 1024 and the Llama-3
vocabulary of 128256 classes)."""

import numpy as np
import pytest
import torch

import oracle
from parity_util import LOSS_RTOL, f64, rel, rel_fro, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def flce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_06_amd as m
    m.load()
    return m


def _logits(rows, V, std, dtype, seed, ld=None):
    g = torch.Generator().manual_seed(seed)
    z = (torch.randn(rows, V, generator=g, dtype=torch.float32) * std).to(dtype)
    t = torch.randint(0, V, (rows,), generator=g, dtype=torch.int32)
    if ld is not None and ld > V:  # rows inside a wider buffer
        buf = torch.zeros(rows, ld, dtype=dtype)
        buf[:, :V] = z
        return buf, t
    return z, t


CASES = [  # rows, V, std, dtype, ld
    (37, 1000, 3.0, torch.bfloat16, None),
    (64, 4099, 8.0, torch.bfloat16, None),    # odd pitch: one logit per lane and step
    (16, 1000, 2.0, torch.bfloat16, 1016),    # pitch > V
    (9, 5, 1.0, torch.bfloat16, None),
    (4, 1, 1.0, torch.bfloat16, None),         # one class: loss 0, gradient 0
    (37, 1000, 3.0, torch.float32, None),
    (5, 40000, 30.0, torch.bfloat16, None),    # large spread: max-shifted sums
    (12, 1003, 2.0, torch.bfloat16, 1008),     # aligned rows, 3 logits past the last 16 bytes
    (40, 16, 1.0, torch.bfloat16, None),       # two 16-byte pieces a row
]


@pytest.mark.parametrize("rows,V,std,dtype,ld", CASES)
def test_cross_entropy_matches_oracle(flce, rows, V, std, dtype, ld):
    zb, t = _logits(rows, V, std, dtype, seed=rows * 13 + V, ld=ld)
    Z = f64(zb[:, :V])
    tt = t.numpy().astype(np.int64)
    exp_rows = oracle.row_losses(Z, tt)
    exp_loss = exp_rows.mean()
    exp_G = oracle.dlogits(Z, tt, rows)
    zfull = zb.cuda()
    z = zfull[:, :V]  # rows of V logits at the buffer's pitch
    say(f"flce_cross_entropy rows={rows} V={V} ld={z.stride(0)} {dtype}")
    row_loss = torch.empty(rows, dtype=torch.float32, device="cuda")
    loss = flce.cross_entropy_(z, t.cuda(), row_loss=row_loss)
    torch.cuda.synchronize()
    G = f64(z[:, :V])
    say(f"  loss {float(loss):.7f} vs {exp_loss:.7f}")
    assert rel(float(loss), exp_loss) <= (1e-6 if exp_loss > 1e-3 else 1e-9) or \
        abs(float(loss) - exp_loss) < 1e-6
    assert np.abs(f64(row_loss) - exp_rows).max() <= 1e-5 * max(1.0, np.abs(exp_rows).max())
    if V == 1:
        assert np.abs(G).max() == 0
        return
    e = rel_fro(G, exp_G)
    say(f"  G rel_fro {e:.2e}")
    assert e <= (4e-3 if dtype == torch.bfloat16 else 1e-5)
    assert np.abs(G.sum(axis=1)).max() <= 1e-2 / rows
    if ld is not None:  # the pitch padding is untouched
        assert torch.count_nonzero(zfull[:, V:]).item() == 0


def test_cross_entropy_llama3_vocab(flce):
    """Page 3's shape: 1024 rows of 128256 bf16 logits (std 2); the loss
    against the oracle over every row, the gradient on sampled rows."""
    rows, V = 1024, 128256
    zb, t = _logits(rows, V, 2.0, torch.bfloat16, seed=7)
    tt = t.numpy().astype(np.int64)
    exp_rows = np.concatenate([oracle.row_losses(f64(zb[i:i + 128]), tt[i:i + 128])
                               for i in range(0, rows, 128)])
    sample = np.array([0, 1, 511, 777, 1023])
    exp_G = oracle.dlogits(f64(zb[sample]), tt[sample], 1) / rows
    z = zb.cuda()
    say("flce_cross_entropy 1024 x 128256 bf16")
    loss = flce.cross_entropy_(z, t.cuda())
    torch.cuda.synchronize()
    el = rel(float(loss), exp_rows.mean())
    eg = rel_fro(f64(z[sample]), exp_G)
    say(f"  loss rel {el:.2e}; sampled G rel_fro {eg:.2e}")
    assert el <= LOSS_RTOL / 100
    assert eg <= 4e-3


def test_cross_entropy_autograd(flce):
    """loss.backward() through the autograd node: the logits' gradient is
    the oracle's times the upstream factor."""
    rows, V = 48, 2048
    zb, t = _logits(rows, V, 3.0, torch.bfloat16, seed=3)
    Z = f64(zb)
    exp_G = oracle.dlogits(Z, t.numpy().astype(np.int64), rows)
    x = zb.cuda().requires_grad_(True)
    say("cross_entropy autograd")
    loss = flce.cross_entropy(x, t.cuda())
    (loss * 0.5).backward()
    torch.cuda.synchronize()
    assert x.grad is not None and x.grad.dtype == torch.bfloat16
    assert rel_fro(f64(x.grad), 0.5 * exp_G) <= 4e-3
