"""Pins for the oracle's bin-local selector (AdaComp page, Abstract and
"Citations in the corpus": fixed-size bins per layer, each bin's largest
|residual| as its threshold, a rate that follows local activity).

The rule the oracle follows: entry i of bin b is sent when v_i != 0 and
|fl32(v_i + u_i)| >= max over the bin of |v_j|; at most cap entries are
delivered, in index order, and only those are masked.  The checks below tie
it to hand-derived values (tests/golden/binlocal_cases.json) and to closed
forms in which the look-ahead is zero (u = 0: the per-bin argmax set), a
doubling (u = v: |v| >= theta/2) or a single entry (L = 1), each computed
with NumPy's segmented maximum instead of the oracle's loops.
"""

import numpy as np
import pytest

from conftest import load_golden


def f32(a):
    return np.asarray(a, dtype=np.float32)


def bits(a):
    return f32(a).view(np.uint32)


def bin_max(absv, L):
    """max |v| per bin of L (ragged last bin), repeated over each bin."""
    starts = np.arange(0, absv.size, L)
    m = np.maximum.reduceat(absv, starts)
    return np.repeat(m, np.diff(np.append(starts, absv.size)))


# ------------------------------------------------------------ hand-derived

@pytest.mark.parametrize("case", load_golden("binlocal_cases.json")["select_cases"],
                         ids=lambda c: c["name"])
def test_binlocal_golden_select(orc, case):
    for cc in case["caps"]:
        u, v = f32(case["u"]).copy(), f32(case["v"]).copy()
        v0, u0 = v.copy(), u.copy()
        idx, val, total = orc.binlocal_select_mask(u, v, case["L"], cc["cap"])
        assert total == len(case["salient"])
        assert idx.tolist() == cc["idx"]
        assert np.array_equal(bits(val), bits(cc["val"]))
        sent = np.zeros(v.size, bool)
        sent[idx] = True
        assert np.all(bits(v[sent]) == 0) and np.all(bits(u[sent]) == 0)
        assert np.array_equal(bits(v[~sent]), bits(v0[~sent]))
        assert np.array_equal(bits(u[~sent]), bits(u0[~sent]))


def test_binlocal_golden_step(orc):
    c = load_golden("binlocal_cases.json")["step_case"]
    g = f32(c["g"])
    u = np.zeros(g.size, np.float32)
    v = f32(c["v0"]).copy()
    idx, val, count, total, norm, scale = orc.binlocal_step(
        c["sizes"], c["L"], c["cap"], g, u, v, 0.9, 0.0)
    assert count.tolist() == c["count"] and total.tolist() == c["total"]
    off = 0
    for t in range(len(c["sizes"])):
        assert idx[off:off + count[t]].tolist() == c["idx"][t]
        assert np.array_equal(bits(val[off:off + count[t]]), bits(c["val"][t]))
        off += c["cap"][t]
    assert np.array_equal(bits(v), bits(c["v_after"]))
    assert np.array_equal(bits(u), bits(c["u_after"]))
    assert scale == np.float32(1.0)


# ------------------------------------------------------------ closed forms

def random_v(rng, n, ties):
    if ties:
        # few distinct magnitudes, random signs, some zeros: many ties
        v = rng.choice(np.array([0.0, 0.125, 0.25, 0.5, 1.0]), n)
        return f32(v * rng.choice([-1.0, 1.0], n))
    return f32(rng.laplace(0, 1e-3, n))


@pytest.mark.parametrize("n,L", [(1, 1), (10, 3), (1000, 50), (1000, 1000),
                                 (1000, 4096), (5003, 64), (20000, 500)])
@pytest.mark.parametrize("ties", [False, True])
def test_binlocal_zero_lookahead_is_bin_argmax(orc, n, L, ties):
    """u = 0: exactly the non-zero entries equal to their bin's max |v|."""
    rng = np.random.default_rng([21, n, L, ties])
    v = random_v(rng, n, ties)
    u = np.zeros(n, np.float32)
    a = np.abs(v.astype(np.float64))
    expect = np.flatnonzero((a > 0) & (a == bin_max(a, L)))
    idx, _, total = orc.binlocal_select_mask(u, v.copy(), L)
    assert idx.tolist() == expect.tolist() and total == expect.size


@pytest.mark.parametrize("n,L", [(1000, 7), (4096, 256), (20000, 500), (30000, 1024)])
@pytest.mark.parametrize("ties", [False, True])
def test_binlocal_doubling_lookahead(orc, n, L, ties):
    """u = v: v + u = 2v exactly, so an entry is sent iff |v| >= theta / 2."""
    rng = np.random.default_rng([22, n, L, ties])
    v = random_v(rng, n, ties)
    a = np.abs(v.astype(np.float64))
    expect = np.flatnonzero((a > 0) & (a >= bin_max(a, L) / 2))
    idx, val, total = orc.binlocal_select_mask(v.copy(), v.copy(), L)
    assert idx.tolist() == expect.tolist() and total == expect.size
    assert np.array_equal(bits(val), bits(v[expect]))


def test_binlocal_single_entry_bins(orc):
    """L = 1: sent iff v != 0 and |v + u| >= |v|; on a grid of multiples of
    2**-8 below 2**8 every binary32 sum is exact, so fp64 decides alike."""
    rng = np.random.default_rng(23)
    n = 50000
    v = f32(rng.integers(-64, 65, n) / 256.0)
    u = f32(rng.integers(-200, 201, n) / 256.0)
    v64, u64 = v.astype(np.float64), u.astype(np.float64)
    expect = np.flatnonzero((v64 != 0) & (np.abs(v64 + u64) >= np.abs(v64)))
    idx, _, total = orc.binlocal_select_mask(u.copy(), v.copy(), 1)
    assert idx.tolist() == expect.tolist() and total == expect.size
    # same-sign updates always qualify, so the rate grows with activity
    same = (v64 * u64 > 0)
    assert np.all(np.isin(np.flatnonzero(same), idx))


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("cap_frac", [0.0, 0.3, 1.0])
def test_binlocal_truncation_and_residual(orc, cap_frac):
    rng = np.random.default_rng([24, int(cap_frac * 10)])
    n, L = 40000, 100
    v0 = random_v(rng, n, False)
    u0 = f32(rng.laplace(0, 1e-3, n))
    full, _, total = orc.binlocal_select_mask(u0.copy(), v0.copy(), L)
    cap = int(cap_frac * total)
    u, v = u0.copy(), v0.copy()
    idx, val, total2 = orc.binlocal_select_mask(u, v, L, cap)
    assert total2 == total
    assert idx.tolist() == full[:cap].tolist()
    # what was sent plus what stays adds up to v before, bitwise
    dense = np.zeros(n, np.float32)
    dense[idx] = val
    assert np.array_equal(bits(dense + v), bits(v0 + np.float32(0)))
    sent = np.zeros(n, bool)
    sent[idx] = True
    assert np.all(bits(u[sent]) == 0)
    assert np.array_equal(bits(u[~sent]), bits(u0[~sent]))


def test_binlocal_step_matches_per_tensor_calls(orc):
    """The step is clip + momentum over the whole gradient, then the
    selector on each tensor on its own (bins restart per tensor)."""
    rng = np.random.default_rng(25)
    sizes = [1, 999, 4096, 70001, 3]
    L = [5, 50, 1024, 333, 1]
    cap = [1, 999, 100, 70001, 0]
    n = sum(sizes)
    g = f32(rng.laplace(0, 1e-2, n))
    u = f32(rng.laplace(0, 1e-3, n))
    v = f32(rng.laplace(0, 1e-3, n))
    u2, v2 = u.copy(), v.copy()
    idx, val, count, total, norm, scale = orc.binlocal_step(
        sizes, L, cap, g, u, v, 0.9, 0.5)
    assert scale < 1
    orc.momentum(g, scale, 0.9, u2, v2)
    off = coff = 0
    for t, nt in enumerate(sizes):
        ut, vt = u2[off:off + nt].copy(), v2[off:off + nt].copy()
        i2, x2, tot2 = orc.binlocal_select_mask(ut, vt, L[t], cap[t])
        assert count[t] == i2.size and total[t] == tot2
        assert np.array_equal(idx[coff:coff + count[t]], i2)
        assert np.array_equal(bits(val[coff:coff + count[t]]), bits(x2))
        assert np.array_equal(bits(u[off:off + nt]), bits(ut))
        assert np.array_equal(bits(v[off:off + nt]), bits(vt))
        off += nt
        coff += cap[t]


def test_binlocal_rejects_bad_arguments(orc):
    z = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        orc.binlocal_select_mask(z.copy(), z.copy(), 0)
    with pytest.raises(ValueError):
        orc.binlocal_select_mask(z.copy(), z.copy(), 2, -1)
    idx, _, total = orc.binlocal_select_mask(z.copy(), z.copy(), 2)
    assert idx.size == 0 and total == 0
