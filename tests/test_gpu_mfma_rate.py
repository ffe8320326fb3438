"""The matrix-core rate microbenchmark (flce_mfma_rate) on the GPU.

It is a measurement aid, so these tests check what it computed and what it
reports rather than a rate:
* zero and all-ones operands give exact results;
* random bf16 operands give what the documented 32x32x16 lane layout
  implies, checked against an fp64 product on the CPU;
* the clock counters agree with the stream's own elapsed time.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def flce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_06_amd as m
    m.load()
    return m


def test_zero_operands_give_zero(flce):
    ops = torch.zeros(8192, dtype=torch.uint8, device="cuda")
    sink, clocks = flce.mfma_rate(ops, 10, 4)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)
    assert torch.all(clocks > 0)


def test_all_ones_is_exact(flce):
    # every product block element is 16 (k = 16 terms of 1 * 1) per round;
    # a wave sums element 0 of its 16 blocks over its 64 lanes
    iters = 100
    ops = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    sink, _ = flce.mfma_rate(ops, iters, 8)
    torch.cuda.synchronize()
    assert torch.all(sink == 64 * 16 * 16 * iters), sink[:4]


def _expected_sink(host, groups, wave, iters):
    """fp64 value of one wave's sink from the documented layout: lane l
    reads group (wave * 64 + l) % groups; pieces 0-3 are A_0..A_3 and 4-7
    are B_0..B_3, lane l holding row (column) l % 32, k = 8 (l // 32) + e;
    element 0 of lane l is D[4 (l // 32)][l % 32] with D = A_i B_j^T."""
    P = host[[(wave * 64 + l) % groups for l in range(64)]]  # [64 lanes, 8 pieces, 8]
    total, scale = 0.0, 0.0
    for i in range(4):
        for j in range(4):
            A = np.zeros((32, 16))
            B = np.zeros((32, 16))
            for l in range(64):
                A[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = P[l, i]
                B[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = P[l, 4 + j]
            D = A @ B.T
            absD = np.abs(A) @ np.abs(B).T
            for l in range(64):
                total += D[4 * (l // 32), l % 32]
                scale += absD[4 * (l // 32), l % 32]
    return iters * total, iters * scale


def test_random_operands_follow_the_lane_layout(flce):
    groups, iters = 256, 8  # 8 waves: the second workgroup wraps onto the same groups
    g = torch.Generator().manual_seed(7)
    x = torch.randn(groups * 64, generator=g).to(torch.bfloat16)
    sink, _ = flce.mfma_rate(x.cuda(), iters, 2)
    torch.cuda.synchronize()
    host = x.double().numpy().reshape(groups, 8, 8)
    got = sink.cpu().double().numpy()
    for w in range(8):
        want, scale = _expected_sink(host, groups, w, iters)
        assert abs(got[w] - want) <= 1e-5 * scale, (w, got[w], want, scale)


def test_clock_counters_agree_with_elapsed_time(flce):
    g = torch.Generator().manual_seed(3)
    ops = torch.randn(1 << 17, generator=g).to(torch.bfloat16).cuda()
    wg = torch.cuda.get_device_properties(0).multi_processor_count
    flce.mfma_rate(ops, 1000, wg)  # warm-up
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    _, clocks = flce.mfma_rate(ops, 20000, wg)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    c = clocks.cpu().double().numpy()
    loop_ms = c[:, 1] / 1e5  # 100 MHz reference ticks
    assert np.all(loop_ms > 0)
    # every wave's loop spans most of the launch and none outlasts it
    assert loop_ms.max() <= ms * 1.02, (loop_ms.max(), ms)
    assert loop_ms.min() >= ms * 0.8, (loop_ms.min(), ms)
    ghz = c[:, 0] / (c[:, 1] * 10.0)  # cycles / (ticks * 10 ns) in GHz
    assert np.all((ghz > 0.5) & (ghz < 3.0)), (ghz.min(), ghz.max())
