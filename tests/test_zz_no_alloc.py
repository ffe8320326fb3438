"""The allocation-free entry point flce_fwd_bwd_noalloc against flce_fwd_bwd.

Both run the same kernels on the same inputs at the same chunk, one over a
caller-provided workspace and one over the library's static device scratch,
so their outputs must agree bit for bit (a stricter form of the parity bar:
loss relative error <= 1e-3, gradients relative Frobenius error <= 1e-2).
Two calls in a row, the second on a smaller input, check that the scratch
keeps no state that a later call depends on; the calls make no allocation
through torch's allocator, a side stream and a captured HIP graph give the
same bits, and sizes beyond the scratch are refused.
"""

import pytest
import torch

from parity_util import GRAD_RTOL, LOSS_RTOL, f64, rel, rel_fro, say
from synth import make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def flce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_06_amd as m
    m.load()  # raises if the HIP library is missing: no fallback exists
    return m


def _run_both(flce, N, H, V, chunk, seed, w_std=0.1, stream=None):
    inp = make_random(N, H, V, dtype="bf16", seed=seed, w_std=w_std)
    h, W, t = inp.h.cuda(), inp.W.cuda(), inp.t.cuda()
    say(f"flce_fwd_bwd N={N} H={H} V={V} chunk={chunk}")
    ref = tuple(x.clone() for x in flce.fwd_bwd(h, W, t, chunk))
    torch.cuda.synchronize()
    loss = torch.full((), float("nan"), dtype=torch.float32, device="cuda")
    gh = torch.full_like(h, float("nan"))
    gw = torch.full((V, H), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.max_memory_allocated()
    say(f"flce_fwd_bwd_noalloc N={N} H={H} V={V} chunk={chunk} "
        f"{'side' if stream is not None else 'current'} stream")
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            got = flce.fwd_bwd_noalloc(h, W, t, chunk, loss=loss, grad_h=gh, grad_W=gw)
    else:
        got = flce.fwd_bwd_noalloc(h, W, t, chunk, loss=loss, grad_h=gh, grad_W=gw)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base  # nothing allocated by the call
    el = rel(float(got[0]), float(ref[0]))
    eh = rel_fro(f64(got[1]), f64(ref[1]))
    ew = rel_fro(f64(got[2]), f64(ref[2]))
    say(f"  loss rel {el:.1e}; grad_h rel_fro {eh:.1e}; grad_W rel_fro {ew:.1e}")
    assert el <= LOSS_RTOL and eh <= GRAD_RTOL and ew <= GRAD_RTOL
    for a, b in zip(got, ref):  # same kernels, same order: the same bits
        assert torch.equal(a, b)


def test_noalloc_matches_fwd_bwd_twice_second_smaller(flce):
    # two 1024-token chunks with 4 grad_h K-split parts each, then a smaller
    # call with a ragged last chunk: what the first call left in the scratch
    # must not leak into the second
    _run_both(flce, 2048, 1024, 32000, 1024, seed=70)
    _run_both(flce, 300, 128, 1000, 128, seed=71, w_std=0.3)


def test_noalloc_on_a_side_stream(flce):
    # a stream other than the null stream: the scratch is looked up on the
    # stream's device, and the call is ordered on that stream
    side = torch.cuda.Stream()
    _run_both(flce, 1000, 256, 4096, 256, seed=72, w_std=0.2, stream=side)


def test_noalloc_under_graph_capture(flce):
    # the callers this entry point is for: one call captured into a HIP graph
    # (nothing allocated while capturing), replayed several times with eager
    # work and synchronisations in between; every replay equals the eager
    # call bit for bit, and a replay after the inputs change in place follows
    # the new inputs
    N, H, V, chunk = 1000, 256, 4096, 256
    a = make_random(N, H, V, dtype="bf16", seed=73, w_std=0.2)
    b = make_random(N, H, V, dtype="bf16", seed=74, w_std=0.2)
    h, W, t = a.h.cuda(), a.W.cuda(), a.t.cuda()
    refs = []
    for inp in (a, b):
        say(f"flce_fwd_bwd (eager reference) N={N} H={H} V={V} chunk={chunk}")
        refs.append(tuple(x.clone() for x in flce.fwd_bwd(inp.h.cuda(), inp.W.cuda(),
                                                          inp.t.cuda(), chunk)))
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    gh = torch.empty_like(h)
    gw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    say("flce_fwd_bwd_noalloc eager warm-up (looks up the scratch address)")
    flce.fwd_bwd_noalloc(h, W, t, chunk, loss=loss, grad_h=gh, grad_W=gw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("flce_fwd_bwd_noalloc captured into a graph")
    with torch.cuda.graph(graph):
        flce.fwd_bwd_noalloc(h, W, t, chunk, loss=loss, grad_h=gh, grad_W=gw)
    torch.cuda.synchronize()
    for rep, which in enumerate((0, 0, 1, 0)):
        src = (a, b)[which]
        h.copy_(src.h.cuda())
        W.copy_(src.W.cuda())
        t.copy_(src.t.cuda())
        for x in (loss, gh, gw):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph replay {rep} (inputs {'ab'[which]})")
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((loss, gh, gw), refs[which]):
            assert torch.equal(got, want)


def test_noalloc_refuses_sizes_beyond_the_scratch(flce):
    N, H, V = 4096, 4096, 128256
    assert flce.workspace_bytes(N, H, V, 2048, torch.bfloat16) > flce.NOALLOC_SCRATCH_BYTES
    h = torch.zeros(N, H, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(V, H, dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(N, dtype=torch.int32, device="cuda")
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    gh = torch.empty_like(h)
    gw = torch.empty((V, H), dtype=torch.float32, device="cuda")
    say("flce_fwd_bwd_noalloc oversize (refused on the host)")
    with pytest.raises(flce.FlceError) as e:
        flce.fwd_bwd_noalloc(h, W, t, 2048, loss=loss, grad_h=gh, grad_W=gw)
    assert e.value.status == 5
