"""Pins for the oracle's hierarchical selector (DGC review, "Research
questions", RQ4: hierarchical thresholding as a runtime strategy for
scalable selection; "Proposed method": only large entries leave).

The rule the oracle follows: level 1 is the sampled threshold theta (the
ceil(S*k/n)-th largest key of the sampled lines); the survivors are the
non-zero entries with key >= theta.  Level 2: when more than k survive, the
k survivors first under (key descending, index ascending) are sent, else all
survivors; in index order, masked.  The count is min(k, survivors).

The checks tie it to hand-derived cases (tests/golden/hier_cases.json), to
the two selectors it must reduce to (exact top-k when at least k survive,
the one-level sampled selector when fewer do; both pinned on their own), to
a full sort on tiny inputs, and to invariants.  Planted mistakes in a NumPy
re-implementation each fail the golden cases.
"""

import numpy as np
import pytest

from conftest import load_golden
from oracle import bruteforce as bf

M32 = np.uint64(0xFFFFFFFF)


def keys(v):
    return np.asarray(v, np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def golden_input(case, n):
    g = np.zeros(n, np.float32)
    for a, b, x in case["segments"]:
        g[a:b] = x
    return g


def golden_expect(case):
    idx = np.concatenate([np.arange(a, b) for a, b in case["idx_ranges"]] or
                         [np.zeros(0, np.int64)])
    val = np.concatenate([np.full(c, x, np.float32) for c, x in case["vals"]] or
                         [np.zeros(0, np.float32)])
    return idx.astype(np.uint32), val.astype(np.float32)


def check_golden(select):
    """select(u, v, k) -> (idx, val, total, theta), in place on u, v.
    Returns the list of problems over the golden cases."""
    c = load_golden("hier_cases.json")
    n = c["n"]
    bad = []
    for case in c["cases"]:
        g = golden_input(case, n)
        u, v = g.copy(), g.copy()  # zero state, momentum: u = v = g
        idx, val, total, theta = select(u, v, case["k"])
        e_idx, e_val = golden_expect(case)
        if idx.tolist() != e_idx.tolist():
            bad.append((case["name"], "idx"))
        if not np.array_equal(bits(val), bits(e_val)):
            bad.append((case["name"], "val"))
        if (len(idx), total, theta) != (case["count"], case["total"], case["theta"]):
            bad.append((case["name"], "counts", len(idx), total, theta))
        res = g.copy()
        res[e_idx] = 0.0
        if not (np.array_equal(bits(u), bits(res)) and np.array_equal(bits(v), bits(res))):
            bad.append((case["name"], "residual"))
    return bad


def test_golden_cases(orc):
    assert check_golden(lambda u, v, k: orc.hier_select_mask(u, v, k, t=5)) == []


def test_golden_step(orc):
    """The same cases through the step (clip off, zero state, m = 0.9): the
    momentum gives u = v = g; the outputs land at offset sum(k[:t])."""
    c = load_golden("hier_cases.json")
    n = c["n"]
    cases = c["cases"]
    g = np.concatenate([golden_input(cs, n) for cs in cases])
    k = [cs["k"] for cs in cases]
    u = np.zeros_like(g)
    v = np.zeros_like(g)
    idx, val, count, total, theta, _, _ = orc.hier_step([n] * len(cases), k, g, u, v,
                                                        0.9, 0.0)
    off = np.concatenate([[0], np.cumsum(k)])
    for t, cs in enumerate(cases):
        e_idx, e_val = golden_expect(cs)
        assert count[t] == cs["count"] and total[t] == cs["total"] and theta[t] == cs["theta"]
        assert idx[off[t]:off[t] + count[t]].tolist() == e_idx.tolist()
        assert np.array_equal(bits(val[off[t]:off[t] + count[t]]), bits(e_val))


# ------------------------------------------------------------ planted mistakes

def np_sample_keys(v, t):
    n = v.size
    lines = -(-n // 32)
    ls = lines if n <= 65536 else min(lines, max(512, lines // 256))
    stride = lines // ls
    j = np.arange(ls, dtype=np.uint64)
    h = ((j * np.uint64(0x9E3779B9)) & M32) ^ np.uint64((t * 0x7F4A7C15) & 0xFFFFFFFF)
    for sh, mul in ((16, 0x85EBCA6B), (13, 0xC2B2AE35)):
        h ^= h >> np.uint64(sh)
        h = (h * np.uint64(mul)) & M32
    h ^= h >> np.uint64(16)
    line = (j * np.uint64(stride) + h % np.uint64(stride)).astype(np.int64)
    el = (line[:, None] * 32 + np.arange(32)[None, :]).ravel()
    return keys(v[el[el < n]]).astype(np.int64)


def np_hier(u, v, k, t=0, *, level2=True, ties_high=False, zeros=False,
            first_in_order=False, from_all=False):
    """A NumPy re-implementation with switches that plant one mistake each."""
    n = v.size
    if k == 0:
        return np.zeros(0, np.uint32), np.zeros(0, np.float32), 0, 0xFFFFFFFF
    sk = np.sort(np_sample_keys(v, t))[::-1]
    J = -(-sk.size * k // n)
    theta = int(sk[J - 1])
    ky = keys(v).astype(np.int64)
    surv = np.flatnonzero((ky >= theta) & ((ky > 0) | zeros))
    pool = np.arange(n) if from_all else surv
    sel = pool
    if level2 and pool.size > k:
        if first_in_order:
            sel = pool[:k]
        else:
            tie = -pool if ties_high else pool
            sel = pool[np.lexsort((tie, -ky[pool]))[:k]]
    sel = np.sort(sel)
    val = v[sel].copy()
    u[sel] = 0.0
    v[sel] = 0.0
    return sel.astype(np.uint32), val, int(surv.size), theta


@pytest.mark.parametrize("mutant", ["no_level2", "ties_high", "zeros_survive",
                                    "first_in_order", "from_all"])
def test_planted_mistakes_fail_the_golden(mutant):
    assert check_golden(np_hier) == []  # the unmutated re-implementation passes
    kw = {"no_level2": dict(level2=False), "ties_high": dict(ties_high=True),
          "zeros_survive": dict(zeros=True), "first_in_order": dict(first_in_order=True),
          "from_all": dict(from_all=True)}[mutant]
    assert check_golden(lambda u, v, k: np_hier(u, v, k, **kw)) != []


# ------------------------------------------------------------ reductions

@pytest.mark.parametrize("n,t", [(1000, 0), (65537, 2), (200003, 3), (1 << 20, 11)])
def test_reduces_to_exact_topk_or_to_level_one(orc, n, t):
    """At least k survivors: the k-th largest key is at or above theta and
    non-zero, so level 2 is exact top-k (orc.select_mask).  Fewer than k:
    level 2 keeps them all, which is the one-level sampled selector without
    a cap.  Both branches must occur over the draws."""
    rng = np.random.default_rng([41, n, t])
    seen = set()
    for trial in range(12):
        if trial % 3 == 2:  # many zeros: theta 0 and short survivor lists
            v = rng.laplace(0, 1e-3, n) * (rng.random(n) < 0.01)
        else:
            v = rng.laplace(0, 1e-3, n) * np.where(rng.random(n) < 0.01, 100.0, 1.0)
        v = v.astype(np.float32)
        k = int(rng.choice([1, max(1, n // 1000), max(1, n // 64), n // 4 + 1, n]))
        u0 = rng.normal(0, 1e-3, n).astype(np.float32)
        uh, vh = u0.copy(), v.copy()
        idx, val, total, theta = orc.hier_select_mask(uh, vh, k, t)
        us, vs = u0.copy(), v.copy()
        s_idx, s_val, s_total, s_theta = orc.sampled_select_mask(us, vs, k, t)
        assert (total, theta) == (s_total, s_theta)
        assert idx.size == min(k, total)
        if total >= k:
            seen.add("exact")
            ue, ve = u0.copy(), v.copy()
            e_idx, e_val = orc.select_mask(ue, ve, k)
            ref = (e_idx, e_val, ue, ve)
        else:
            seen.add("level1")
            ref = (s_idx, s_val, us, vs)
        assert idx.tolist() == ref[0].tolist()
        assert np.array_equal(bits(val), bits(ref[1]))
        assert np.array_equal(bits(uh), bits(ref[2])) and np.array_equal(bits(vh), bits(ref[3]))
    if n > 65536:
        assert seen == {"exact", "level1"}, seen


@pytest.mark.parametrize("n", [1, 7, 33, 64])
def test_tiny_inputs_against_a_full_sort(orc, n):
    """Up to 65536 elements the sample is the whole tensor and theta the exact
    k-th largest key: the result is the full sort's top k when at least k
    entries are non-zero, else every non-zero entry."""
    rng = np.random.default_rng([42, n])
    for trial in range(20):
        v = (rng.choice([0.0, 0.5, 1.0, 2.0], n) * rng.choice([-1, 1], n)).astype(np.float32)
        for k in range(0, n + 1):
            idx, _, _, _ = orc.hier_select_mask(np.zeros(n, np.float32), v.copy(), k)
            nz = np.flatnonzero(v != 0)
            want = bf.topk_fullsort(v, k) if nz.size >= k else nz
            assert idx.tolist() == [int(x) for x in want], (trial, k)


def test_count_never_exceeds_k(orc):
    """Laplace entries, n = 2**22, k = n/1000 and n/64: the count is min(k,
    survivors), so never above k, and the survivors are the sampled count
    (within +-40% of k)."""
    n = 1 << 22
    for seed in range(3):
        v = np.random.default_rng([43, seed]).laplace(0, 1e-3, n).astype(np.float32)
        for k in (n // 1000 + 1, n // 64):
            idx, _, total, _ = orc.hier_select_mask(np.zeros(n, np.float32), v.copy(), k, seed)
            assert idx.size == min(k, total) and idx.size <= k
            assert 0.6 * k <= total <= 1.4 * k


def test_rejects_bad_k(orc):
    v = np.ones(10, np.float32)
    for k in (-1, 11):
        with pytest.raises(ValueError):
            orc.hier_select_mask(np.zeros(10, np.float32), v.copy(), k)
    with pytest.raises(ValueError):
        orc.hier_step([10], [11], v, np.zeros(10, np.float32), v.copy(), 0.9, 0.0)
