"""Pins for the oracle's shared-index (commutative) compression.

Source: the ScaleComp abstract on the taxoreview.com page -- the learners'
gradient distributions are alike, which allows a commutative compressor
whose communication cost stays constant in the number of learners and which
an all-reduce can carry.  The page gives no mechanism; the reading the oracle
follows: each step one learner, the leader (step mod W), takes its exact
top-k per tensor (the DGC rule); every learner sends its v at that shared
index set and masks u and v there; the aggregate is the learner-order sum of
the value vectors (K floats, whatever W), scattered into the dense sum.

The checks tie it to hand-derived steps (tests/golden/shared_cases.json), to
the defining property (compressing the sum of the learners' v equals summing
their compressed values, checked where binary32 addition is exact), to the
DGC selection it reduces to for the leader, to the oracle's own stream
encoder and decoder, to a sequential NumPy float32 sum whose order is
visible in the bits, and to the residual invariants.  Planted mistakes in a
NumPy re-implementation each fail one of the checks.
"""

import numpy as np
import pytest

from conftest import load_golden


def f32(a):
    return np.asarray(a, dtype=np.float32)


def bits(a):
    return f32(a).view(np.uint32)


# ------------------------------------------------------------ hand-derived

def run_golden(impl_step, impl_sum, leader_of):
    """Replays the golden steps with the given implementation: impl_step(g,
    u, v, m, idx) -> (vals) for a learner taking index set idx (in place on
    u, v) and impl_sum(list of vals) -> sum.  Returns the list of problems."""
    import oracle
    c = load_golden("shared_cases.json")
    W, n, k, m = c["learners"], c["n"], c["k"], c["momentum"]
    u = [np.zeros(n, np.float32) for _ in range(W)]
    v = [np.zeros(n, np.float32) for _ in range(W)]
    bad = []
    for st in c["steps"]:
        L = leader_of(st["step"], W)
        if L != st["leader"]:
            bad.append(("leader", st["step"], L))
        # the leader: DGC's exact top-k (clip off)
        idx, lval, _, _ = oracle.step([n], [k], f32(st["g"][L]), u[L], v[L], m, 0.0)
        if idx.tolist() != st["idx"]:
            bad.append(("idx", st["step"], idx.tolist()))
        vals = []
        for w in range(W):
            if w == L:
                vals.append(lval)
            else:
                vals.append(impl_step(f32(st["g"][w]), u[w], v[w], m, idx))
        for w in range(W):
            if not np.array_equal(bits(vals[w]), bits(st["vals"][w])):
                bad.append(("vals", st["step"], w, vals[w].tolist()))
            if not np.array_equal(bits(u[w]), bits(st["u"][w])):
                bad.append(("u", st["step"], w, u[w].tolist()))
            if not np.array_equal(bits(v[w]), bits(st["v"][w])):
                bad.append(("v", st["step"], w, v[w].tolist()))
        s = impl_sum(vals)
        if not np.array_equal(bits(s), bits(st["sum"])):
            bad.append(("sum", st["step"], s.tolist()))
        dense = np.zeros(n, np.float32)
        dense[idx] = s
        if not np.array_equal(bits(dense), bits(st["dense"])):
            bad.append(("dense", st["step"]))
    return bad


def oracle_follower(g, u, v, m, idx):
    import oracle
    val, _, _ = oracle.shared_step([g.size], [idx.size], idx, g, u, v, m, 0.0)
    return val


def test_shared_golden_steps(orc):
    assert run_golden(oracle_follower, orc.shared_sum, lambda t, W: t % W) == []


# Planted mistakes, each in a NumPy re-implementation of one part: every one
# must be caught by the golden steps.
def _np_follower(g, u, v, m, idx, *, mask=True, before_update=False, shift=0):
    if before_update:
        val = v[idx].copy()
    u[:] = f32(f32(np.float32(m) * u) + g)
    v[:] = f32(v + u)
    if not before_update:
        val = v[np.minimum(idx + shift, v.size - 1)].copy()
    if mask:
        u[idx] = 0.0
        v[idx] = 0.0
    return val


def _np_sum(vals, reverse=False):
    s = np.zeros(vals[0].size, np.float32)
    for x in (vals[::-1] if reverse else vals):
        s = f32(s + x)
    return s


@pytest.mark.parametrize("mutant", ["no_mask", "value_before_update", "index_shift",
                                    "sum_reversed", "fixed_leader"])
def test_planted_mistakes_fail_the_golden(orc, mutant):
    follower, summ, leader = _np_follower, _np_sum, (lambda t, W: t % W)
    if mutant == "no_mask":
        follower = lambda *a: _np_follower(*a, mask=False)  # noqa: E731
    elif mutant == "value_before_update":
        follower = lambda *a: _np_follower(*a, before_update=True)  # noqa: E731
    elif mutant == "index_shift":
        follower = lambda *a: _np_follower(*a, shift=1)  # noqa: E731
    elif mutant == "sum_reversed":
        summ = lambda vals: _np_sum(vals, reverse=True)  # noqa: E731
    elif mutant == "fixed_leader":
        leader = lambda t, W: 0  # noqa: E731
    # the unmutated NumPy re-implementation passes
    assert run_golden(_np_follower, _np_sum, lambda t, W: t % W) == []
    assert run_golden(follower, summ, leader) != []


# ------------------------------------------------------------ properties

def test_sum_follows_learner_order(orc):
    """Binary32 addition is not associative: with 1, 2^-24, -1 the learner
    order gives (1 + 2^-24) - 1 = 0 (the tie rounds to even), the reverse
    order gives 2^-24; the oracle's sum is the sequential one from +0.0."""
    a = f32([1.0, -0.0, 3.0])
    b = f32([2.0 ** -24, -0.0, 1e-8])
    c = f32([-1.0, -0.0, -3.0])
    s = orc.shared_sum([a, b, c])
    want = f32(f32(f32(np.float32(0.0) + a) + b) + c)
    assert np.array_equal(bits(s), bits(want))
    assert s[0] == 0.0 and bits(s)[1] == 0  # +0 + -0 = +0
    rev = orc.shared_sum([c, b, a])
    assert rev[0] == np.float32(2.0 ** -24)


@pytest.mark.parametrize("W", [1, 2, 3, 8])
def test_commutes_with_the_sum_over_learners(orc, W):
    """The defining property: compressing the learners' summed v at the
    shared set gives the sum of the learners' compressed values.  Integer
    values keep every binary32 sum exact, so the order of additions cannot
    hide a mistake in the gather."""
    rng = np.random.default_rng([41, W])
    n, k = 5000, 37
    vs = [f32(rng.integers(-1000, 1000, n)) for _ in range(W)]
    idx = np.sort(rng.choice(n, k, replace=False)).astype(np.uint32)
    vals = [orc.shared_gather_mask(np.zeros(n, np.float32), v.copy(), idx) for v in vs]
    total = np.zeros(n, np.float32)
    for v in vs:
        total = f32(total + v)
    compressed_sum = orc.shared_gather_mask(np.zeros(n, np.float32), total, idx)
    assert np.array_equal(bits(orc.shared_sum(vals)), bits(compressed_sum))
    # the aggregate holds K values whatever the number of learners
    assert orc.shared_sum(vals).size == k


@pytest.mark.parametrize("seed", range(4))
def test_leader_rule_is_dgc_top_k(orc, seed):
    """A learner whose index set is its own exact top-k gets exactly what
    DGC's select + mask gives: the leader's path and the shared path agree."""
    rng = np.random.default_rng([42, seed])
    n = int(rng.choice([1000, 70001]))
    k = max(1, n // int(rng.choice([10, 1000])))
    v = f32(rng.laplace(0, 1e-3, n))
    if seed % 2:
        v[rng.random(n) < 0.3] = np.float32(1e-3)  # ties
    u = f32(rng.laplace(0, 1e-3, n))
    u1, v1 = u.copy(), v.copy()
    idx, val = orc.select_mask(u1, v1, k)
    u2, v2 = u.copy(), v.copy()
    val2 = orc.shared_gather_mask(u2, v2, idx)
    assert np.array_equal(bits(val), bits(val2))
    assert np.array_equal(bits(u1), bits(u2)) and np.array_equal(bits(v1), bits(v2))


@pytest.mark.parametrize("seed", range(3))
def test_dense_sum_equals_decoding_every_learners_stream(orc, seed):
    """Scattering the learner-order sum at the shared set gives the same bits
    as encoding each learner's (shared indices, values) stream and decoding
    the W streams in learner order onto +0.0 (the oracle's encoder and
    decoder, an independent path; gaps above 65535 need fillers)."""
    rng = np.random.default_rng([43, seed])
    n, k, W = 300007, 211, 4
    idx = np.sort(rng.choice(n, k, replace=False)).astype(np.uint32)
    idx[-1] = n - 1
    vals = [f32(rng.standard_normal(k)) for _ in range(W)]
    vals[1][::5] = -0.0
    s = orc.shared_sum(vals)
    dense = np.zeros(n, np.float32)
    dense[idx] = s
    want = np.zeros(n, np.float32)
    for x in vals:
        r, vv = orc.encode(idx, x)
        assert orc.decode_accumulate(r, vv, want) == 0
    assert np.array_equal(bits(dense), bits(want))


def test_follower_residual_invariants(orc):
    """sent + residual == accumulated v bitwise (disjoint supports), u = +0
    exactly at the shared set and untouched elsewhere."""
    rng = np.random.default_rng(44)
    sizes = [70001, 1, 4096, 300007]
    n = sum(sizes)
    k = [71, 1, 5, 301]
    g = f32(rng.laplace(0, 1e-2, n))
    u = f32(rng.laplace(0, 1e-3, n))
    v = f32(rng.laplace(0, 1e-3, n))
    # the leader's index set, from another gradient
    ul, vl = u.copy(), v.copy()
    idx, _, _, _ = orc.step(sizes, k, f32(rng.laplace(0, 1e-2, n)), ul, vl, 0.9, 0.5)
    u0, v0 = u.copy(), v.copy()
    val, norm, s = orc.shared_step(sizes, k, idx, g, u, v, 0.9, 0.5)
    norm2, s2 = orc.clip_scale(g, 0.5)
    assert norm == norm2 and s == s2
    orc.momentum(g, s, 0.9, u0, v0)  # the accumulated state before masking
    off = np.concatenate([[0], np.cumsum(sizes)])
    koff = np.concatenate([[0], np.cumsum(k)])
    sent = np.zeros(n, np.float32)
    mask = np.zeros(n, bool)
    for t in range(len(sizes)):
        gi = off[t] + idx[koff[t]:koff[t + 1]].astype(np.int64)
        sent[gi] = val[koff[t]:koff[t + 1]]
        mask[gi] = True
    assert np.array_equal(bits(f32(sent + v)), bits(f32(v0 + np.float32(0.0))))
    assert np.all(bits(u[mask]) == 0) and np.all(bits(v[mask]) == 0)
    assert np.array_equal(bits(u[~mask]), bits(u0[~mask]))
    assert np.array_equal(bits(v[~mask]), bits(v0[~mask]))


def test_rejects_bad_index_sets(orc):
    z = np.zeros(10, np.float32)
    for bad in ([3, 3], [5, 2], [10], [0, 11]):
        with pytest.raises(ValueError):
            orc.shared_gather_mask(z.copy(), z.copy(), np.array(bad, np.uint32))
    assert orc.shared_gather_mask(z.copy(), z.copy(), np.zeros(0, np.uint32)).size == 0
