"""Pins for the oracle's sampled-threshold selector (DGC review, "Research
questions", RQ4: hierarchical thresholding for scalable selection; "Proposed
method": only large entries leave).

The rule the oracle follows: sample whole 32-element lines of the tensor
(all lines up to 65536 elements, else max(512, lines/256) of them, one per
stride segment, placed by MurmurHash3's fmix32); theta = the ceil(S*k/n)-th
largest sampled key; send every non-zero entry with key >= theta, at most cap
of them in index order.  The checks tie it to fmix32's published test
vectors, to exact top-k when the sample is the whole tensor, to a sample
drawn independently in NumPy with the threshold taken by np.sort, to the
statistics of a quantile estimate, and to invariants.
"""

import numpy as np
import pytest

from oracle import bruteforce as bf

M32 = np.uint64(0xFFFFFFFF)


def keys(v):
    return np.asarray(v, np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)


def np_fmix32(h):
    h = np.asarray(h, np.uint64) & M32
    h ^= h >> np.uint64(16)
    h = (h * np.uint64(0x85EBCA6B)) & M32
    h ^= h >> np.uint64(13)
    h = (h * np.uint64(0xC2B2AE35)) & M32
    h ^= h >> np.uint64(16)
    return h


def np_sample_lines(n, t):
    lines = -(-n // 32)
    ls = lines if n <= 65536 else min(lines, max(512, lines // 256))
    stride = lines // ls
    j = np.arange(ls, dtype=np.uint64)
    x = ((j * np.uint64(0x9E3779B9)) & M32) ^ np.uint64((t * 0x7F4A7C15) & 0xFFFFFFFF)
    return (j * np.uint64(stride) + np_fmix32(x) % np.uint64(stride)).astype(np.int64), stride


def test_fmix32_published_vectors(orc):
    """MurmurHash3_x86_32 of the empty input is fmix32(seed); its published
    values for seeds 0, 1 and 0xFFFFFFFF are 0, 0x514E28B7, 0x81F16F39."""
    assert orc.fmix32(0) == 0
    assert orc.fmix32(1) == 0x514E28B7
    assert orc.fmix32(0xFFFFFFFF) == 0x81F16F39
    xs = np.random.default_rng(31).integers(0, 1 << 32, 200, dtype=np.uint64)
    assert [orc.fmix32(int(x)) for x in xs] == np_fmix32(xs).tolist()


@pytest.mark.parametrize("n", [1, 31, 1000, 65536])
def test_whole_tensor_sample_is_exact_topk_with_ties(orc, n):
    """Up to 65536 elements the sample is the tensor: theta is the exact
    k-th largest key, so the sent set is the top k plus any further entries
    tied with it (zeros never)."""
    rng = np.random.default_rng([32, n])
    for trial in range(4):
        if trial < 2:
            v = rng.laplace(0, 1e-3, n).astype(np.float32)      # distinct keys
        else:
            v = (rng.choice([0.0, 0.25, 0.5, 1.0], n) * rng.choice([-1, 1], n)).astype(np.float32)
        k = int(rng.integers(1, n + 1))
        ky = keys(v).astype(np.int64)
        T = int(np.sort(ky)[::-1][k - 1])
        expect = np.flatnonzero((ky >= T) & (ky > 0))
        idx, val, total, theta = orc.sampled_select_mask(np.zeros(n, np.float32), v.copy(), k)
        assert theta == T
        assert idx.tolist() == expect.tolist() and total == expect.size
        if trial < 2:
            assert idx.tolist() == bf.topk_fullsort(v, k).tolist()


@pytest.mark.parametrize("n,t", [(65537, 0), (200003, 3), (1 << 22, 17), (1 << 24, 63)])
def test_threshold_matches_an_independent_sample(orc, n, t):
    """The sample drawn in NumPy from the same definition: one line per stride
    segment, distinct; theta = np.sort of its keys at rank ceil(S*k/n)."""
    rng = np.random.default_rng([33, n])
    v = rng.laplace(0, 1e-3, n).astype(np.float32)
    lines, stride = np_sample_lines(n, t)
    seg = lines // stride
    assert np.array_equal(seg[seg < lines.size], np.arange(lines.size)[seg < lines.size])
    assert np.unique(lines).size == lines.size
    el = (lines[:, None] * 32 + np.arange(32)[None, :]).ravel()
    el = el[el < n]
    sk = np.sort(keys(v[el]).astype(np.int64))[::-1]
    for k in (1, n // 1000 + 1, n // 64, n):
        J = -(-el.size * k // n)
        ky = keys(v).astype(np.int64)
        idx, _, total, theta = orc.sampled_select_mask(np.zeros(n, np.float32), v.copy(), k, t)
        assert theta == sk[J - 1], (k, J)
        assert total == int(((ky >= theta) & (ky > 0)).sum())
        assert idx.size == total


def test_count_follows_k_within_sampling_error(orc):
    """Laplace entries, n = 2**24, k = n/1000: S = 65536 samples, about 66
    above the true threshold; the sent count is within +-40% of k (more than
    3 standard deviations of the quantile estimate) for every seed, and
    within 10% on average."""
    n, k = 1 << 24, 16778
    ratios = []
    for seed in range(6):
        v = np.random.default_rng([34, seed]).laplace(0, 1e-3, n).astype(np.float32)
        _, _, total, _ = orc.sampled_select_mask(np.zeros(n, np.float32), v, k, seed, cap=0)
        ratios.append(total / k)
    assert all(0.6 < r < 1.4 for r in ratios), ratios
    assert abs(np.mean(ratios) - 1) < 0.1, ratios


def test_threshold_falls_and_count_grows_with_k(orc):
    v = np.random.default_rng(35).laplace(0, 1e-3, 300001).astype(np.float32)
    last_theta, last_total = 1 << 32, -1
    for k in (1, 30, 300, 3000, 30000, 300001):
        _, _, total, theta = orc.sampled_select_mask(np.zeros(v.size, np.float32),
                                                     v.copy(), k, 2, cap=0)
        assert theta <= last_theta and total >= last_total
        last_theta, last_total = theta, total


@pytest.mark.parametrize("cap_frac", [0.0, 0.5, 1.0])
def test_truncation_and_residual(orc, cap_frac):
    rng = np.random.default_rng([36, int(cap_frac * 2)])
    n, k = 300001, 3000
    v0 = rng.laplace(0, 1e-3, n).astype(np.float32)
    u0 = rng.laplace(0, 1e-3, n).astype(np.float32)
    full, _, total, _ = orc.sampled_select_mask(u0.copy(), v0.copy(), k, 5)
    cap = int(cap_frac * total)
    u, v = u0.copy(), v0.copy()
    idx, val, total2, _ = orc.sampled_select_mask(u, v, k, 5, cap)
    assert total2 == total and idx.tolist() == full[:cap].tolist()
    dense = np.zeros(n, np.float32)
    dense[idx] = val
    assert np.array_equal(keys(dense + v), keys(v0 + np.float32(0)))
    assert np.array_equal((dense + v).view(np.uint32), (v0 + np.float32(0)).view(np.uint32))
    sent = np.zeros(n, bool)
    sent[idx] = True
    assert np.all(u[sent].view(np.uint32) == 0)
    assert np.array_equal(u[~sent].view(np.uint32), u0[~sent].view(np.uint32))


def test_step_matches_per_tensor_calls(orc):
    """Clip + momentum over the whole gradient, then each tensor sampled
    with its own index t."""
    rng = np.random.default_rng(37)
    sizes = [1, 70001, 4096, 300007, 0]
    k = [1, 71, 4096, 301, 0]
    cap = [1, 100, 4096, 200, 0]
    n = sum(sizes)
    g = rng.laplace(0, 1e-2, n).astype(np.float32)
    u = rng.laplace(0, 1e-3, n).astype(np.float32)
    v = rng.laplace(0, 1e-3, n).astype(np.float32)
    u2, v2 = u.copy(), v.copy()
    idx, val, count, total, theta, norm, scale = orc.sampled_step(sizes, k, cap, g, u, v,
                                                                  0.9, 0.5)
    orc.momentum(g, scale, 0.9, u2, v2)
    off = coff = 0
    for t, nt in enumerate(sizes):
        ut, vt = u2[off:off + nt].copy(), v2[off:off + nt].copy()
        i2, x2, tot2, th2 = orc.sampled_select_mask(ut, vt, k[t], t, cap[t])
        assert count[t] == i2.size and total[t] == tot2 and theta[t] == th2
        assert np.array_equal(idx[coff:coff + count[t]], i2)
        assert np.array_equal(val[coff:coff + count[t]].view(np.uint32), x2.view(np.uint32))
        assert np.array_equal(u[off:off + nt].view(np.uint32), ut.view(np.uint32))
        assert np.array_equal(v[off:off + nt].view(np.uint32), vt.view(np.uint32))
        off += nt
        coff += cap[t]


def test_rejects_bad_arguments(orc):
    z = np.zeros(10, np.float32)
    with pytest.raises(ValueError):
        orc.sampled_select_mask(z.copy(), z.copy(), 11)
    with pytest.raises(ValueError):
        orc.sampled_select_mask(z.copy(), z.copy(), -1)
    with pytest.raises(ValueError):
        orc.sampled_select_mask(z.copy(), z.copy(), 1, 0, -1)
    idx, _, total, theta = orc.sampled_select_mask(z.copy(), z.copy(), 0)
    assert idx.size == 0 and total == 0 and theta == 0xFFFFFFFF
    # all zero: theta 0, but zeros are never sent
    idx, _, total, theta = orc.sampled_select_mask(z.copy(), z.copy(), 5)
    assert idx.size == 0 and total == 0 and theta == 0


@pytest.mark.parametrize("seed", range(4))
def test_sampled_and_exact_sets_are_nested(orc, seed):
    """Both selections are threshold sets ({key >= theta} and top-k, i.e.
    {key > T} plus the lowest-index ties at T), so one contains the other
    and they differ in exactly |count - k| entries, all between the two
    thresholds: the deviation from exact top-k is measured by the count."""
    rng = np.random.default_rng([38, seed])
    n = int(rng.choice([70001, 1 << 20]))
    k = n // int(rng.choice([4, 64, 1000]))
    v = rng.laplace(0, 1e-3, n).astype(np.float32)
    if seed % 2:
        v[rng.random(n) < 0.3] = 0.0
    ex, _ = orc.select_mask(np.zeros(n, np.float32), v.copy(), k)
    sm, _, total, theta = orc.sampled_select_mask(np.zeros(n, np.float32), v.copy(), k, seed)
    a, b = set(ex.tolist()), set(sm.tolist())
    assert a <= b or b <= a
    assert len(a ^ b) == abs(total - k)
    ky = keys(v).astype(np.int64)
    lo, hi = sorted([int(theta), int(np.sort(ky)[::-1][k - 1])])
    for i in a ^ b:
        assert lo <= ky[i] <= hi
