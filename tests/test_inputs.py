"""The seeded input generator: determinism, shapes, dtypes and distributions."""

import dataclasses
import math

import numpy as np
import torch

from synth import CONFIGS, make_inputs, make_random, to_float64


def _small(cfg, **kw):
    return dataclasses.replace(cfg, **kw)


def test_configs_match_the_workloads():
    shapes = {c.idx: (c.N, c.H, c.V, c.dtype) for c in CONFIGS.values()}
    assert shapes == {
        1: (256, 128, 1000, "f32"),
        2: (2048, 4096, 32000, "bf16"),
        3: (8192, 4096, 128256, "bf16"),
        4: (16384, 4096, 128256, "bf16"),
        5: (8192, 3584, 256000, "bf16"),
    }
    assert CONFIGS[3].flops == 6 * 8192 * 4096 * 128256
    assert CONFIGS[4].naive_logits_bytes == 4 * 16384 * 128256


def test_same_seed_same_bits():
    cfg = CONFIGS[1]
    a = make_inputs(cfg, seed=0)
    b = make_inputs(cfg, seed=0)
    c = make_inputs(cfg, seed=1)
    assert torch.equal(a.h, b.h) and torch.equal(a.W, b.W) and torch.equal(a.t, b.t)
    assert not torch.equal(a.h, c.h)
    assert a.h.dtype == torch.float32 and a.t.dtype == torch.int32


def test_block_threads_do_not_change_bits():
    cfg = _small(CONFIGS[2], N=3000, H=64, V=2500)
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    assert torch.equal(a.W.view(torch.int16), b.W.view(torch.int16))
    assert a.h.dtype == torch.bfloat16


def test_bf16_is_round_to_nearest_even_of_fp32():
    cfg = _small(CONFIGS[2], N=64, H=32, V=100)
    x = make_inputs(cfg)
    f = _small(cfg, dtype="f32")
    y = make_inputs(f)
    assert torch.equal(y.h.to(torch.bfloat16), x.h)
    assert torch.equal(y.W.to(torch.bfloat16), x.W)


def test_moments():
    x = make_inputs(_small(CONFIGS[2], N=2048, H=256, V=4096))
    h, W = to_float64(x.h), to_float64(x.W)
    assert abs(h.mean()) < 0.01 and abs(h.std() - 1) < 0.01
    assert abs(W.std() - 0.02) < 0.0005
    t = x.t.numpy()
    assert t.min() >= 0 and t.max() < 4096
    assert abs(t.mean() - 4095 / 2) < 0.05 * 4096


def test_rms_normalised_rows():
    x = make_inputs(_small(CONFIGS[3], N=64, H=512, V=100))
    h = to_float64(x.h)
    ms = np.mean(h * h, axis=1)
    assert np.all(np.abs(ms - 1) < 1e-2)


def test_outliers_and_zipf():
    cfg = _small(CONFIGS[5], N=1024, H=512, V=256000)
    x = make_inputs(cfg)
    h = to_float64(x.h)
    big = np.mean(np.abs(h) > 8.0)
    # a scaled entry exceeds 8 when |x| > 0.4 (probability 0.689)
    assert abs(big - 0.001 * 0.689) < 0.0003
    t = x.t.numpy()
    zeta = np.sum(np.arange(1, 256001, dtype=np.float64) ** -1.1)
    p0 = 1.0 / zeta
    assert abs(np.mean(t == 0) - p0) < 4 * math.sqrt(p0 * (1 - p0) / 1024)
    assert t.max() < 256000 and t.min() >= 0


def test_make_random_shapes():
    x = make_random(3, 8, 5, dtype="bf16", seed=3)
    assert x.h.shape == (3, 8) and x.W.shape == (5, 8) and x.t.shape == (3,)
    assert x.N == 3 and x.H == 8 and x.V == 5
