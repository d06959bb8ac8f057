"""Pins for the CPU oracle: each check ties it to something other than
itself -- values derived by hand from the DGC review page's "Proposed
method" rules (tests/golden), closed forms, library routines, brute force on
tiny inputs, and invariants that any correct result must satisfy.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import load_golden
from oracle import bruteforce as bf


def bits_to_f32(hexes):
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


def f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------- clipping

@pytest.mark.parametrize("n", [1, 7, 65536, 65537, 300001])
def test_clip_norm_matches_linalg(orc, n):
    g = np.random.default_rng([11, n]).laplace(0, 1e-3, n).astype(np.float32)
    norm, _ = orc.clip_scale(g, 0.0)
    ref = float(np.linalg.norm(g.astype(np.float64)))
    # each side's recursive binary64 sum of n positive terms is within
    # n * 2**-53 (relative) of the exact sum
    assert abs(norm - ref) <= 2 * n * 2.0 ** -53 * ref


def test_clip_norm_matches_correctly_rounded_sum(orc):
    g = np.random.default_rng(12).standard_normal(200003).astype(np.float32)
    norm, _ = orc.clip_scale(g, 0.0)
    # squares of binary32 values are exact in binary64; fsum rounds the
    # exact sum once
    S = math.fsum(float(x) * float(x) for x in g.astype(np.float64))
    # recursive summation of n positive terms: relative error <= n * 2**-53
    # in S, half of that in sqrt(S), plus the rounding of sqrt
    assert abs(norm - math.sqrt(S)) <= (g.size / 2 + 1) * 2.0 ** -53 * math.sqrt(S)


def test_clip_three_four_five(orc):
    g = np.array([3.0, 4.0], np.float32)
    assert orc.clip_scale(g, 2.5) == (5.0, np.float32(0.5))
    # norm equal to the threshold: not above it, so no scaling
    assert orc.clip_scale(g, 5.0) == (5.0, np.float32(1.0))
    assert orc.clip_scale(g, 4.99)[1] == np.float32(4.99 / 5.0)
    # clip <= 0 means off
    assert orc.clip_scale(g, 0.0)[1] == np.float32(1.0)
    assert orc.clip_scale(g, -1.0)[1] == np.float32(1.0)


def test_clip_power_of_two_exact(orc):
    # 4**5 ones: norm 32 exactly; c = 0.5 gives s = 2**-6 exactly
    g = np.ones(4 ** 5, np.float32)
    norm, s = orc.clip_scale(g, 0.5)
    assert norm == 32.0 and s == np.float32(2.0 ** -6)
    u = np.zeros_like(g)
    v = np.zeros_like(g)
    orc.momentum(g, s, 0.9, u, v)
    assert np.all(u == np.float32(2.0 ** -6)) and np.all(v == u)


def test_clipped_norm_is_threshold(orc):
    g = np.random.default_rng(13).laplace(0, 1e-2, 100000).astype(np.float32)
    c = 0.5
    norm, s = orc.clip_scale(g, c)
    assert norm > c
    u = np.zeros_like(g)
    v = np.zeros_like(g)
    orc.momentum(g, s, 0.9, u, v)  # from zero state u = fl32(g*s)
    clipped = float(np.linalg.norm(u.astype(np.float64)))
    # one rounding of s plus one rounding per product
    assert abs(clipped - c) <= 2.0 ** -22 * c


# ---------------------------------------------------------------- momentum

def test_momentum_from_zero_state_is_scaled_gradient(orc):
    g = np.random.default_rng(14).laplace(0, 1e-3, 4099).astype(np.float32)
    for s in (np.float32(1.0), np.float32(0.3)):
        u = np.zeros_like(g)
        v = np.zeros_like(g)
        orc.momentum(g, s, 0.9, u, v)
        assert np.array_equal(f32_bits(u), f32_bits(g * s))
        assert np.array_equal(f32_bits(v), f32_bits(u))


@pytest.mark.parametrize("scale", [1.0, 0.25])
def test_momentum_dyadic_closed_form(orc, scale):
    """With m = 1/2, a power-of-two scale and small dyadic gradients every
    intermediate is exact in binary32, so the recurrence must equal its
    unrolled closed form: u_t = sum_{j<=t} m^(t-j) s g_j, v_t = sum_{j<=t} u_j."""
    rng = np.random.default_rng(15)
    n, T, m = 257, 6, Fraction(1, 2)
    gs = [(rng.integers(-4096, 4097, n) / 256.0).astype(np.float32) for _ in range(T)]
    u = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(T):
        orc.momentum(gs[t], np.float32(scale), 0.5, u, v)
        for i in range(0, n, 37):
            ut = sum(m ** (t - j) * Fraction(float(gs[j][i])) * Fraction(scale)
                     for j in range(t + 1))
            vt = sum(sum(m ** (tau - j) * Fraction(float(gs[j][i])) * Fraction(scale)
                         for j in range(tau + 1)) for tau in range(t + 1))
            assert Fraction(float(u[i])) == ut
            assert Fraction(float(v[i])) == vt


def _f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def test_momentum_binary32_rounding(orc):
    """m = 0.9f: each product and sum rounded once to binary32.  Binary64
    holds the exact product of two binary32 numbers, and rounding a binary64
    sum of two binary32 numbers to binary32 is correctly rounded, so Python
    floats plus one explicit rounding give the exact expected bits."""
    rng = np.random.default_rng(16)
    n = 2000
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    u = rng.laplace(0, 1e-3, n).astype(np.float32)
    v = rng.laplace(0, 1e-2, n).astype(np.float32)
    u0, v0 = u.copy(), v.copy()
    s = np.float32(0.7)
    orc.momentum(g, s, 0.9, u, v)
    m = _f32(0.9)
    for i in range(n):
        gs = _f32(float(g[i]) * float(s))
        un = _f32(_f32(m * float(u0[i])) + gs)
        vn = _f32(float(v0[i]) + un)
        assert float(u[i]) == un and float(v[i]) == vn


# ---------------------------------------------------------------- selection

def test_select_golden_ties(orc):
    gold = load_golden("select_cases.json")
    v0 = bits_to_f32(gold["v"])
    assert np.array_equal(v0, np.array(gold["v_decimal"], np.float32))
    for case in gold["cases"]:
        v = v0.copy()
        u = np.ones_like(v)
        idx, val = orc.select_mask(u, v, case["k"])
        assert idx.tolist() == case["idx"], case
        assert np.array_equal(f32_bits(val), f32_bits(v0[idx]))
        assert np.all(f32_bits(v[idx]) == 0) and np.all(f32_bits(u[idx]) == 0)
        rest = np.setdiff1d(np.arange(v.size), idx)
        assert np.array_equal(f32_bits(v[rest]), f32_bits(v0[rest]))
        assert np.all(u[rest] == 1.0)


def _tricky_vector(rng, n):
    kind = rng.integers(0, 4)
    if kind == 0:
        return rng.laplace(0, 1e-3, n).astype(np.float32)
    if kind == 1:  # few distinct magnitudes: many ties
        pool = np.array([0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 2.0], np.float32)
        return pool[rng.integers(0, pool.size, n)]
    if kind == 2:  # mostly zeros of both signs
        x = np.zeros(n, np.float32)
        x[rng.random(n) < 0.5] = -0.0
        hot = rng.random(n) < 0.05
        x[hot] = rng.standard_normal(int(hot.sum())).astype(np.float32)
        return x
    # denormals and huge values
    x = rng.standard_normal(n).astype(np.float32)
    x[rng.random(n) < 0.2] = np.float32(1e-45) * rng.integers(1, 4, 1)[0]
    x[rng.random(n) < 0.01] = np.float32(3e38)
    return x


@pytest.mark.parametrize("seed", range(60))
def test_select_matches_full_sort(orc, seed):
    rng = np.random.default_rng([17, seed])
    n = int(rng.integers(1, 3000))
    v0 = _tricky_vector(rng, n)
    for k in {0, 1, n, int(rng.integers(0, n + 1)), max(0, n // 1000)}:
        v = v0.copy()
        u = np.ones_like(v)
        idx, val = orc.select_mask(u, v, k)
        assert np.array_equal(idx, bf.topk_fullsort(v0, k))
        assert np.array_equal(f32_bits(val), f32_bits(v0[idx]))


def test_select_python_brute_force_tiny(orc):
    rng = np.random.default_rng(18)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        v0 = np.array(rng.choice([0.0, -0.0, 1.0, -1.0, 2.0, 0.5], n), np.float32)
        k = int(rng.integers(0, n + 1))
        order = sorted(range(n), key=lambda i: (-abs(float(v0[i])), i))
        want = sorted(order[:k])
        idx, _ = orc.select_mask(np.zeros_like(v0), v0.copy(), k)
        assert idx.tolist() == want


def test_select_invariants_large(orc):
    rng = np.random.default_rng(19)
    n = 1 << 20
    v0 = rng.laplace(0, 1e-3, n).astype(np.float32)
    v0[rng.integers(0, n, 5000)] = np.float32(0.0069)  # a block of ties
    u0 = rng.laplace(0, 1e-3, n).astype(np.float32)
    for k in (1049, 20000, n // 4):
        u, v = u0.copy(), v0.copy()
        idx, val = orc.select_mask(u, v, k)
        assert idx.size == k and np.all(np.diff(idx.astype(np.int64)) > 0)
        keys = bf.magnitude_keys(v0)
        sel = np.zeros(n, bool)
        sel[idx] = True
        kmin = keys[sel].min()
        assert kmin >= keys[~sel].max()
        ties_in = np.flatnonzero(sel & (keys == kmin))
        ties_out = np.flatnonzero(~sel & (keys == kmin))
        if ties_out.size:
            assert ties_in.max() < ties_out.min()
        # masking: u and v are +0.0 on the sent set and untouched elsewhere
        assert np.all(f32_bits(u[sel]) == 0) and np.all(f32_bits(v[sel]) == 0)
        assert np.array_equal(f32_bits(u[~sel]), f32_bits(u0[~sel]))
        # sent + residual == accumulated v, bitwise (disjoint supports)
        dense = np.zeros(n, np.float32)
        dense[idx] = val
        assert np.array_equal(f32_bits(dense + v), f32_bits(v0 + np.float32(0)))
        # the magnitudes agree with a library top-k
        tk = torch.topk(torch.from_numpy(np.abs(v0)), k).values.numpy()
        assert np.array_equal(np.sort(np.abs(val)), np.sort(tk))


def test_select_rejects_bad_k(orc):
    v = np.ones(4, np.float32)
    with pytest.raises(ValueError):
        orc.select_mask(np.zeros_like(v), v, 5)
    with pytest.raises(ValueError):
        orc.select_mask(np.zeros_like(v), v, -1)


# ---------------------------------------------------------------- encoding

def _expand(pairs):
    out = []
    for x, cnt in pairs:
        out += [x] * cnt
    return out


def test_encode_golden(orc):
    gold = load_golden("encode_cases.json")
    for case in gold["cases"]:
        idx = np.array(case["idx"], np.uint32)
        val = bits_to_f32(case["val"])
        runs_w = case["runs"] if "runs" in case else _expand(case["runs_repeat"])
        vals_w = case["vals"] if "vals" in case else _expand(case["vals_repeat"])
        runs, vals = orc.encode(idx, val)
        assert runs.tolist() == runs_w, case["name"]
        assert np.array_equal(f32_bits(vals), f32_bits(bits_to_f32(vals_w))), case["name"]
        # decoding onto zeros gives back 0 + value at each index
        dense = np.zeros(case["n"], np.float32)
        assert orc.decode_accumulate(runs, vals, dense) == 0
        want = np.zeros(case["n"], np.float32)
        want[idx] = np.float32(0.0) + val
        assert np.array_equal(f32_bits(dense), f32_bits(want)), case["name"]


@pytest.mark.parametrize("seed", range(20))
def test_encode_matches_walk(orc, seed):
    rng = np.random.default_rng([20, seed])
    n = int(rng.integers(1, 300000))
    dens = [0.5, 0.01, 1e-4, 5e-6][seed % 4]
    sel = np.flatnonzero(rng.random(n) < dens).astype(np.uint32)
    if seed % 5 == 0 and n > 1:
        sel = np.unique(np.concatenate([sel, [0, n - 1]])).astype(np.uint32)
    val = rng.standard_normal(sel.size).astype(np.float32)
    runs, vals = orc.encode(sel, val)
    r2, v2 = bf.encode_walk(n, sel, val)
    assert np.array_equal(runs, r2) and np.array_equal(f32_bits(vals), f32_bits(v2))
    # closed form: E = k + sum floor(G / 65536)
    gaps = np.diff(np.concatenate([[-1], sel.astype(np.int64)])) - 1
    assert runs.size == sel.size + int((gaps // 65536).sum())


def test_encode_capacity_and_order_errors(orc):
    with pytest.raises(ValueError):
        orc.encode(np.array([70000], np.uint32), np.ones(1, np.float32), cap=1)
    with pytest.raises(ValueError):
        orc.encode(np.array([5, 5], np.uint32), np.ones(2, np.float32))


def test_compression_ratio_flat1m(orc):
    """2**20 Laplace entries at 99.9% sparsity: k = 1049 entries of 6 bytes
    (no gap reaches 65536), 4 MiB / (6 * 1049) = 666.4x."""
    n = 1 << 20
    k = orc.k_for_density(n, 1, 1000)
    assert k == 1049
    v = np.random.default_rng(21).laplace(0, 1e-3, n).astype(np.float32)
    idx, val = orc.select_mask(np.zeros_like(v), v, k)
    runs, vals = orc.encode(idx, val)
    assert runs.size == k
    assert round(4 * n / (6 * runs.size), 1) == 666.4


# ---------------------------------------------------------------- decoding

def test_decode_matches_add_at(orc):
    rng = np.random.default_rng(22)
    n = 200000
    streams = []
    for w in range(4):
        sel = np.flatnonzero(rng.random(n) < 0.003).astype(np.uint32)
        sel = np.unique(np.concatenate([sel, rng.integers(0, n, 3)])).astype(np.uint32)
        val = rng.standard_normal(sel.size).astype(np.float32)
        streams.append(orc.encode(sel, val))
    dense = np.zeros(n, np.float32)
    for runs, vals in streams:
        assert orc.decode_accumulate(runs, vals, dense) == 0
    want = bf.decode_accumulate_addat(streams, n)
    assert np.array_equal(f32_bits(dense), f32_bits(want))


def test_decode_flags_corrupt_stream(orc):
    dense = np.zeros(10, np.float32)
    runs = np.array([3, 4, 5], np.uint16)  # positions 3, 8, 14 > 9
    vals = np.ones(3, np.float32)
    assert orc.decode_accumulate(runs, vals, dense) == -1
    assert dense[3] == 1 and dense[8] == 1


# ---------------------------------------------------------------- k schedule

def test_k_schedule_exact_rationals(orc):
    n = 350_000_000
    ks = [orc.k_for_density(n, 1, d) for d in (4, 16, 64, 250, 1000)]
    assert ks == [87_500_000, 21_875_000, 5_468_750, 1_400_000, 350_000]
    # binary floating point would give 350,001 for the last one
    assert math.ceil(n * (1 - 0.999)) == 350_001
    for nn in (1, 999, 1000, 1001, 2 ** 24, 2 ** 20):
        assert orc.k_for_density(nn, 1, 1000) == math.ceil(Fraction(nn, 1000))
    assert orc.k_for_density(1 << 24, 1, 1000) == 16778


# ---------------------------------------------------------------- composite

def test_step_equals_composition(orc):
    rng = np.random.default_rng(23)
    sizes = np.array([64, 1000, 4097, 1], np.int64)
    k = np.array([1, 1, 5, 1], np.int64)
    n = int(sizes.sum())
    g = rng.laplace(0, 1e-2, n).astype(np.float32)
    u0 = rng.laplace(0, 1e-3, n).astype(np.float32)
    v0 = rng.laplace(0, 1e-3, n).astype(np.float32)
    u1, v1 = u0.copy(), v0.copy()
    idx, val, norm, s = orc.step(sizes, k, g, u1, v1, 0.9, 0.5)
    u2, v2 = u0.copy(), v0.copy()
    norm2, s2 = orc.clip_scale(g, 0.5)
    orc.momentum(g, s2, 0.9, u2, v2)
    off = np.concatenate([[0], np.cumsum(sizes)])
    parts_i, parts_v = [], []
    for t in range(sizes.size):
        i_t, v_t = orc.select_mask(u2[off[t]:off[t + 1]], v2[off[t]:off[t + 1]], k[t])
        parts_i.append(i_t)
        parts_v.append(v_t)
    assert (norm, s) == (norm2, s2)
    assert np.array_equal(idx, np.concatenate(parts_i))
    assert np.array_equal(f32_bits(val), f32_bits(np.concatenate(parts_v)))
    assert np.array_equal(f32_bits(u1), f32_bits(u2))
    assert np.array_equal(f32_bits(v1), f32_bits(v2))
