"""Shared driver for the GPU parity tests: runs the HIP path (through the
C ABI) and the CPU oracle on the same seeded inputs and compares them."""

from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence

import numpy as np

import oracle
from sparsified_gradient_compression_amd import dgc


def oracle_k(n, density):
    """k for a tensor of n elements at an exact density, from the oracle's
    own warm-up schedule; the library's (dgc_k_for_density) must agree."""
    from fractions import Fraction
    d = Fraction(density)
    k = oracle.k_for_density(n, d.numerator, d.denominator)
    assert dgc.k_for_density(n, d) == k, (n, d)
    return k


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def first_diff(a: np.ndarray, b: np.ndarray) -> str:
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    bad = np.flatnonzero(a != b)
    if bad.size == 0:
        return "equal"
    i = int(bad[0])
    return f"{bad.size} differ; first at {i}: {a[i]!r} vs {b[i]!r}"


@dataclass
class StepResult:
    idx: np.ndarray
    val: np.ndarray
    norm: float
    scale: np.float32


@dataclass
class Pair:
    """One learner on both sides: the GPU learner and the oracle's u, v."""
    sizes: List[int]
    k_max: List[int]
    momentum: float = 0.9
    learner: Optional[dgc.Learner] = None
    u: np.ndarray = field(default=None)
    v: np.ndarray = field(default=None)

    def __post_init__(self):
        n = int(sum(self.sizes))
        self.learner = dgc.Learner(self.sizes, self.k_max, self.momentum)
        self.u = np.zeros(n, np.float32)
        self.v = np.zeros(n, np.float32)

    def step(self, g: np.ndarray, k: Sequence[int], clip: float, check_state=True,
             tag=""):
        import torch
        L = self.learner
        gd = torch.from_numpy(g).cuda()
        idx, val = L.compress(gd, k, clip)
        torch.cuda.synchronize()
        got = StepResult(idx.cpu().numpy().view(np.uint32).copy(),
                         val.cpu().numpy().copy(), float(L.norm.cpu()[0]),
                         np.float32(L.scale.cpu()[0]))
        o_idx, o_val, o_norm, o_s = oracle.step(np.array(self.sizes), np.array(k),
                                                g, self.u, self.v, self.momentum, clip)
        assert L.status() == dgc.DGC_OK, f"{tag}: device status"
        if clip > 0:
            assert abs(got.norm - o_norm) <= 1e-6 * o_norm, (tag, got.norm, o_norm)
        else:
            assert got.norm == -1.0
        assert got.scale == o_s, (tag, "scale", got.scale, o_s)
        assert np.array_equal(got.idx, o_idx), (tag, "idx", first_diff(got.idx, o_idx))
        assert np.array_equal(f32_bits(got.val), f32_bits(o_val)), (
            tag, "val", first_diff(f32_bits(got.val), f32_bits(o_val)))
        if check_state:
            gu = L.u[: len(self.u)].cpu().numpy()
            gv = L.v[: len(self.v)].cpu().numpy()
            assert np.array_equal(f32_bits(gu), f32_bits(self.u)), (
                tag, "u", first_diff(f32_bits(gu), f32_bits(self.u)))
            assert np.array_equal(f32_bits(gv), f32_bits(self.v)), (
                tag, "v", first_diff(f32_bits(gv), f32_bits(self.v)))
        return got, (o_idx, o_val)


def oracle_streams(sizes, k, idx, val):
    """Encode per tensor with the oracle; returns lists of (runs, vals)."""
    out = []
    koff = np.concatenate([[0], np.cumsum(k)])
    for t in range(len(sizes)):
        i = idx[koff[t]:koff[t + 1]]
        v = val[koff[t]:koff[t + 1]]
        cap = int(k[t]) + int(sizes[t]) // 65536
        out.append(oracle.encode(i, v, cap=max(cap, 1)))
    return out


def gpu_streams(pair: Pair, k):
    """The GPU learner's encoded streams split per tensor (host copies)."""
    import torch
    runs, vals, entries = pair.learner.encode(k)
    torch.cuda.synchronize()
    cap = pair.learner.cap
    r = runs.cpu().numpy().view(np.uint16)
    v = vals.cpu().numpy()
    e = entries.cpu().numpy()
    out = []
    for t in range(len(pair.sizes)):
        out.append((r[cap[t]:cap[t] + e[t]].copy(), v[cap[t]:cap[t] + e[t]].copy()))
    return out


def compare_streams(got, want, tag=""):
    for t, ((gr, gv), (wr, wv)) in enumerate(zip(got, want)):
        assert np.array_equal(gr, wr), (tag, t, "runs", first_diff(gr, wr))
        assert np.array_equal(f32_bits(gv), f32_bits(wv)), (tag, t, "vals")
