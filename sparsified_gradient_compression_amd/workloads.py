"""Seeded synthetic workloads: tensor shapes, schedules and gradient draws.

This module is the one place that both the HIP path and the CPU oracle take
their inputs from.  It holds data and random draws only -- none of the
compressor's arithmetic (no clipping, momentum, selection, encoding, and no
k computation: densities are kept as exact fractions and each side turns
them into k on its own).

The DGC review page ("Deep Gradient Compression: Reducing the Communication
Bandwidth for Distributed Training", Abstract and Key findings) measures on
CIFAR-10, ImageNet, Penn Treebank and LibriSpeech with ResNet and DeepSpeech
models; seeded draws of the same tensor shapes stand in for those trained
gradients here.

Recipe (every draw in binary64, cast once to binary32 with round to nearest
even):

* a generator ``numpy.random.default_rng([cfg, learner, step, tensor,
  block])`` for each 2**24-element block of each tensor;
* Laplace(0, b): ``b * E * sign`` with ``E = standard_exponential(m)`` drawn
  first, then ``ceil(m/8)`` random bytes whose bits (``unpackbits``, most
  significant first) give the sign, bit 1 meaning negative;
* per-tensor Laplace scales ``b_t = 10 ** U(-5, -2)`` from
  ``default_rng([cfg, 1_000_000, tensor]).uniform(-5, -2)``;
* the heavy-tailed normal: ``standard_normal(m) * sigma`` drawn first, then
  ``random(m) < 0.01`` selects the entries multiplied by 100.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from fractions import Fraction
from typing import Optional, Sequence, Tuple

import numpy as np

BLOCK = 1 << 24


# --------------------------------------------------------------------------
# Model shapes
# --------------------------------------------------------------------------

def resnet50_shapes() -> Tuple[Tuple[str, Tuple[int, ...]], ...]:
    """Parameter tensors of ResNet-50 in definition order (torchvision
    layout): stem conv, then 16 bottleneck blocks in stages of (3, 4, 6, 3)
    with widths (64, 128, 256, 512) and expansion 4, a 1x1 downsample conv
    + BN in each stage's first block, BN weight and bias per conv, and the
    1000-way classifier."""
    out = [("conv1.weight", (64, 3, 7, 7)), ("bn1.weight", (64,)),
           ("bn1.bias", (64,))]
    inplanes = 64
    for stage, (planes, blocks) in enumerate(((64, 3), (128, 4), (256, 6),
                                              (512, 3)), start=1):
        for b in range(blocks):
            p = f"layer{stage}.{b}."
            out += [
                (p + "conv1.weight", (planes, inplanes, 1, 1)),
                (p + "bn1.weight", (planes,)), (p + "bn1.bias", (planes,)),
                (p + "conv2.weight", (planes, planes, 3, 3)),
                (p + "bn2.weight", (planes,)), (p + "bn2.bias", (planes,)),
                (p + "conv3.weight", (planes * 4, planes, 1, 1)),
                (p + "bn3.weight", (planes * 4,)),
                (p + "bn3.bias", (planes * 4,)),
            ]
            if b == 0:
                out += [
                    (p + "downsample.0.weight", (planes * 4, inplanes, 1, 1)),
                    (p + "downsample.1.weight", (planes * 4,)),
                    (p + "downsample.1.bias", (planes * 4,)),
                ]
            inplanes = planes * 4
    out += [("fc.weight", (1000, 2048)), ("fc.bias", (1000,))]
    return tuple(out)


def deepspeech_shapes() -> Tuple[Tuple[str, Tuple[int, ...]], ...]:
    """A DeepSpeech-sized recurrent model: two 2-D convolutions, five
    bidirectional GRU layers with hidden sizes (1152, 1152, 1152, 1280, 1280)
    whose gate matrices are 3H x In and 3H x H per direction (In = 32*41 for
    the first layer, else twice the previous hidden size), and a 29-way
    output layer."""
    out = [("conv1.weight", (32, 1, 41, 11)), ("conv2.weight", (32, 32, 21, 11))]
    hidden = (1152, 1152, 1152, 1280, 1280)
    inp = 32 * 41
    for layer, h in enumerate(hidden):
        for d in ("fwd", "bwd"):
            out += [(f"gru{layer}.{d}.w_ih", (3 * h, inp)),
                    (f"gru{layer}.{d}.w_hh", (3 * h, h))]
        inp = 2 * h
    out += [("fc.weight", (29, 2 * hidden[-1]))]
    return tuple(out)


def _numel(shape: Sequence[int]) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """One workload: tensor sizes, per-step densities, learners, clipping.

    ``densities[t]`` is the fraction of each tensor sent at step t, as an
    exact ``Fraction``; ``clip`` is the clipping threshold (0 = off);
    ``dist`` names the gradient distribution.
    """
    name: str
    cfg_id: int
    sizes: Tuple[int, ...]
    densities: Tuple[Fraction, ...]
    learners: int
    clip: float
    momentum: float
    dist: str
    laplace_b: float = 1e-3
    sigma: float = 1e-3

    @property
    def n(self) -> int:
        return int(sum(self.sizes))

    @property
    def steps(self) -> int:
        return len(self.densities)


# Clipping threshold c * N**-1/2 with c = 1 and N = 4 learners.
CLIP_N4 = 1.0 * 4 ** -0.5
MOMENTUM = 0.9


def _make_workloads():
    rn50 = tuple(_numel(s) for _, s in resnet50_shapes())
    ds = tuple(_numel(s) for _, s in deepspeech_shapes())
    return {
        "flat1m": Workload("flat1m", 1, (1 << 20,), (Fraction(1, 1000),), 1,
                           0.0, MOMENTUM, "laplace"),
        "resnet50": Workload("resnet50", 2, rn50, (Fraction(1, 1000),) * 10,
                             1, CLIP_N4, MOMENTUM, "laplace_logscale"),
        "deepspeech": Workload("deepspeech", 3, ds, (Fraction(1, 1000),), 4,
                               CLIP_N4, MOMENTUM, "normal_heavy"),
        "warmup350m": Workload("warmup350m", 4, (350_000_000,),
                               (Fraction(1, 4), Fraction(1, 16),
                                Fraction(1, 64), Fraction(1, 250),
                                Fraction(1, 1000)), 1, 0.0, MOMENTUM,
                               "laplace"),
        "flat1b": Workload("flat1b", 5, (1 << 24,) * 64,
                           (Fraction(1, 1000),) * 3, 4, CLIP_N4, MOMENTUM,
                           "laplace_logscale"),
    }


WORKLOADS = _make_workloads()


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(wl: Workload, factor: int, name: Optional[str] = None) -> Workload:
    """The same workload with every tensor size divided by ``factor``
    (rounded up, at least 1): a small stand-in with the same tensor count,
    distribution and schedule."""
    sizes = tuple(max(1, -(-s // factor)) for s in wl.sizes)
    return Workload(name or f"{wl.name}/{factor}", wl.cfg_id, sizes,
                    wl.densities, wl.learners, wl.clip, wl.momentum, wl.dist,
                    wl.laplace_b, wl.sigma)


# --------------------------------------------------------------------------
# Draws
# --------------------------------------------------------------------------

def tensor_scales(cfg_id: int, n_tensors: int) -> np.ndarray:
    """Per-tensor Laplace scales, log-uniform in [1e-5, 1e-2]."""
    out = np.empty(n_tensors, np.float64)
    for t in range(n_tensors):
        out[t] = 10.0 ** np.random.default_rng([cfg_id, 1_000_000, t]).uniform(-5.0, -2.0)
    return out


def laplace_draw(rng: np.random.Generator, m: int, b: float) -> np.ndarray:
    e = rng.standard_exponential(m)
    bits = np.unpackbits(rng.integers(0, 256, (m + 7) // 8, dtype=np.uint8))[:m]
    return (b * e * (1.0 - 2.0 * bits)).astype(np.float32)


def normal_heavy_draw(rng: np.random.Generator, m: int, sigma: float) -> np.ndarray:
    z = rng.standard_normal(m) * sigma
    heavy = rng.random(m) < 0.01
    z[heavy] *= 100.0
    return z.astype(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gradient(wl: Workload, learner: int, step: int,
             out: Optional[np.ndarray] = None) -> np.ndarray:
    """The float32 gradient of ``learner`` at ``step``: all tensors end to
    end.  Generated in parallel over 2**24-element blocks."""
    n = wl.n
    if out is None:
        out = np.empty(n, np.float32)
    assert out.dtype == np.float32 and out.size == n
    scales = tensor_scales(wl.cfg_id, len(wl.sizes)) if wl.dist == "laplace_logscale" else None
    jobs = []
    off = 0
    for t, s in enumerate(wl.sizes):
        for blk, lo in enumerate(range(0, s, BLOCK)):
            jobs.append((t, blk, off + lo, min(BLOCK, s - lo)))
        off += s

    def run(job):
        t, blk, start, m = job
        rng = np.random.default_rng([wl.cfg_id, learner, step, t, blk])
        if wl.dist == "laplace":
            out[start:start + m] = laplace_draw(rng, m, wl.laplace_b)
        elif wl.dist == "laplace_logscale":
            out[start:start + m] = laplace_draw(rng, m, float(scales[t]))
        elif wl.dist == "normal_heavy":
            out[start:start + m] = normal_heavy_draw(rng, m, wl.sigma)
        else:
            raise ValueError(wl.dist)

    if len(jobs) == 1 or n < (1 << 22):
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(run, jobs))
    return out
