"""The seeded workloads: shapes against the DGC review page's model sizes,
determinism of the draws, and the shape of their distributions."""

import math
from fractions import Fraction

import numpy as np

from conftest import load_golden
from sparsified_gradient_compression_amd import workloads as W


def test_model_sizes_match_page():
    gold = load_golden("model_sizes.json")
    rn = W.get("resnet50")
    assert rn.n == gold["resnet50"]["params"]
    assert len(rn.sizes) == gold["resnet50"]["tensors"]
    assert round(rn.n * 4 / 2 ** 20) == gold["resnet50"]["mib_rounded"]
    # 53 convolutions: stem + 16 blocks x 3 + 4 downsample
    convs = [s for name, s in W.resnet50_shapes() if len(s) == 4]
    assert len(convs) == 53
    assert min(rn.sizes) == 64 and max(rn.sizes) == 2_359_296
    assert sum(1 for s in rn.sizes if s < 1000) == 84
    ds = W.get("deepspeech")
    assert ds.n == gold["deepspeech"]["params"]
    assert len(ds.sizes) == gold["deepspeech"]["tensors"]
    assert round(ds.n * 4 / 1e6) == gold["deepspeech"]["mb_rounded"]
    assert abs(ds.n * 4 / 1e6 - gold["deepspeech"]["page_mb"]) < 1.0


def test_workload_table():
    assert W.get("flat1m").n == 1 << 20
    assert W.get("warmup350m").densities == tuple(
        Fraction(1, d) for d in (4, 16, 64, 250, 1000))
    big = W.get("flat1b")
    assert big.n == 1 << 30 and len(big.sizes) == 64
    assert big.learners == 4 and big.steps == 3 and big.clip == 0.5
    assert W.get("deepspeech").learners == 4


def test_draws_are_deterministic_and_distinct():
    wl = W.scaled(W.get("resnet50"), 100)
    a = W.gradient(wl, 0, 0)
    b = W.gradient(wl, 0, 0)
    c = W.gradient(wl, 1, 0)
    d = W.gradient(wl, 0, 1)
    assert a.dtype == np.float32 and a.size == wl.n
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_laplace_draw_moments():
    x = W.laplace_draw(np.random.default_rng(1), 1 << 20, 1e-3).astype(np.float64)
    # Laplace(0, b): mean 0, E|x| = b, P(|x| > t) = exp(-t/b)
    assert abs(x.mean()) < 5e-6
    assert abs(np.abs(x).mean() - 1e-3) < 1e-5
    tail = np.mean(np.abs(x) > 1e-3 * math.log(1000))
    assert abs(tail - 1e-3) < 2e-4


def test_normal_heavy_draw():
    x = W.normal_heavy_draw(np.random.default_rng(2), 1 << 20, 1e-3).astype(np.float64)
    frac_big = np.mean(np.abs(x) > 0.01)  # |z| > 10 sigma only for scaled ones
    assert 0.0085 < frac_big < 0.0105


def test_logscale_tensor_scales():
    s = W.tensor_scales(5, 64)
    assert np.all(s >= 1e-5) and np.all(s <= 1e-2)
    assert np.array_equal(s, W.tensor_scales(5, 64))


def test_parallel_generation_matches_serial():
    wl = W.Workload("t", 9, (3 << 23, 5), (Fraction(1, 1000),), 1, 0.0, 0.9,
                    "laplace")
    par = W.gradient(wl, 0, 0)
    ser = np.concatenate([
        W.laplace_draw(np.random.default_rng([9, 0, 0, 0, 0]), 1 << 24, 1e-3),
        W.laplace_draw(np.random.default_rng([9, 0, 0, 0, 1]), (3 << 23) - (1 << 24), 1e-3),
        W.laplace_draw(np.random.default_rng([9, 0, 0, 1, 0]), 5, 1e-3),
    ])
    assert np.array_equal(par, ser)
