"""GPU parity of hierarchical thresholding (DGC review, "Research
questions", RQ4): dgc_compress_hier + dgc_encode_counts + decode through the
C ABI against the CPU oracle, bit for bit on the sent counts, indices,
values, u/v state, streams and dense sums.

The first level is the sampled threshold, the second an exact select among
its survivors.  Layouts cover whole-tensor samples (<= 65536 elements) and
line samples, unaligned tensor starts, ragged tails, k from 0 to n, the
per-tensor kernels and the spread passes (DGC_OPT_SELECT_GRID), the forced
whole-tensor select (DGC_OPT_SELECT_PATH), lists of at most k survivors sent
whole, longer lists selected from, and pieces whose survivors overflow their
slots (then the select runs on the whole tensor under the floor).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from gpu_harness import f32_bits, first_diff, oracle_k, say
from sparsified_gradient_compression_amd import dgc
from sparsified_gradient_compression_amd import workloads as W
from test_gpu_binlocal import check_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dgc.lib()
    return torch


class HierPair:
    def __init__(self, sizes, k_max, momentum=0.9, path=0, grid=0):
        self.sizes = [int(s) for s in sizes]
        self.learner = dgc.Learner(self.sizes, k_max, momentum)
        self.learner.set_option(dgc.DGC_OPT_SELECT_PATH, path)
        self.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
        n = sum(self.sizes)
        self.u = np.zeros(n, np.float32)
        self.v = np.zeros(n, np.float32)
        self.m = momentum
        self.seen = set()

    def step(self, g, k, clip, tag=""):
        import torch
        assert g.size == sum(self.sizes), (tag, g.size)
        lr = self.learner
        idx, val, count = lr.compress_hier(torch.from_numpy(g).cuda(), k, clip)
        torch.cuda.synchronize()
        g_idx = idx.cpu().numpy().view(np.uint32)
        g_val = val.cpu().numpy()
        g_cnt = count.cpu().numpy()
        info = lr.select_info()
        o_idx, o_val, o_cnt, o_tot, o_th, o_norm, o_s = oracle.hier_step(
            self.sizes, k, g, self.u, self.v, self.m, clip)
        assert lr.status() == dgc.DGC_OK, (tag, "status")
        assert np.array_equal(g_cnt, o_cnt), (tag, "count", first_diff(g_cnt, o_cnt))
        assert (g_cnt <= np.asarray(k)).all(), tag
        for t, kt in enumerate(k):
            if kt == 0:
                continue
            mode = int(info[t, 0])
            self.seen.add(("dense",) if mode == 2 else
                          ("list", "whole" if o_cnt[t] == o_tot[t] else "select"))
            if mode == 1:  # the list: the survivors, from the floor max(theta, 1)
                assert info[t, 1] == max(int(o_th[t]), 1), (tag, t, info[t, 1], o_th[t])
                assert info[t, 2] == o_tot[t], (tag, t, "survivors", info[t, 2], o_tot[t])
        if clip > 0:
            norm = float(lr.norm.cpu()[0])
            assert abs(norm - o_norm) <= 1e-6 * o_norm, (tag, norm, o_norm)
        assert np.float32(lr.scale.cpu()[0]) == o_s, (tag, "scale")
        off = 0
        for t, kt in enumerate(k):
            a, b = off, off + int(o_cnt[t])
            assert np.array_equal(g_idx[a:b], o_idx[a:b]), (tag, t, "idx",
                                                            first_diff(g_idx[a:b], o_idx[a:b]))
            assert np.array_equal(f32_bits(g_val[a:b]), f32_bits(o_val[a:b])), (tag, t, "val")
            off += int(kt)
        gu = lr.u[: len(self.u)].cpu().numpy()
        gv = lr.v[: len(self.v)].cpu().numpy()
        assert np.array_equal(f32_bits(gu), f32_bits(self.u)), (
            tag, "u", first_diff(f32_bits(gu), f32_bits(self.u)))
        assert np.array_equal(f32_bits(gv), f32_bits(self.v)), (
            tag, "v", first_diff(f32_bits(gv), f32_bits(self.v)))
        return o_idx, o_val, o_cnt

    def check_encode(self, k, o_idx, o_val, o_cnt, tag=""):
        import torch
        runs, vals, entries = self.learner.encode_counts(k)
        torch.cuda.synchronize()
        assert self.learner.status() == dgc.DGC_OK, (tag, "encode status")
        scap = self.learner.cap
        r = runs.cpu().numpy().view(np.uint16)
        v = vals.cpu().numpy()
        e = entries.cpu().numpy()
        want = []
        off = 0
        for t, nt in enumerate(self.sizes):
            wr, wv = oracle.encode(o_idx[off:off + o_cnt[t]], o_val[off:off + o_cnt[t]],
                                   cap=max(int(k[t]) + nt // 65536, 1))
            assert e[t] == wr.size, (tag, t, "entries")
            assert np.array_equal(r[scap[t]:scap[t] + e[t]], wr), (tag, t, "runs")
            assert np.array_equal(f32_bits(v[scap[t]:scap[t] + e[t]]), f32_bits(wv)), (tag, t)
            want.append((wr, wv))
            off += int(k[t])
        return want


def run(sizes, ks, grads, clip, learners=1, path=0, grid=0, k_max=None, tag=""):
    """ks[step]: per-tensor lists; grads(w, step) -> float32[n].  Returns
    the union of the (source, kind) cases the steps went through."""
    if k_max is None:
        k_max = [max(ks[s][t] for s in range(len(ks))) for t in range(len(sizes))]
    pairs = [HierPair(sizes, k_max, path=path, grid=grid) for _ in range(learners)]
    for step, k in enumerate(ks):
        streams = []
        for w, p in enumerate(pairs):
            say(f"{tag} step {step} learner {w} T={len(sizes)} n={sum(sizes)}")
            o_idx, o_val, o_cnt = p.step(grads(w, step), k, clip, tag=f"{tag} s{step} w{w}")
            streams.append(p.check_encode(k, o_idx, o_val, o_cnt, tag=f"{tag} s{step} w{w}"))
        check_decode(pairs, streams, sizes, tag=f"{tag} s{step}")
    return set().union(*(p.seen for p in pairs))


GRIDS = [(0, 0), (0, 2), (1, 0), (1, 2)]  # (select path, select grid)


@pytest.mark.parametrize("path,grid", GRIDS)
def test_flat1m(path, grid):
    wl = W.get("flat1m")
    n = wl.n
    k = [oracle_k(n, wl.densities[0])]
    run([n], [k, k, k], lambda w, s: W.gradient(wl, w, s), 0.0, path=path, grid=grid,
        tag=f"flat1m p{path} g{grid}")


@pytest.mark.parametrize("path,grid", GRIDS)
def test_resnet50_layout_scaled(path, grid):
    """161 tensors scaled 1/8: whole-tensor samples and line samples,
    k = ceil(n/1000), clipping on, three steps."""
    wl = W.scaled(W.get("resnet50"), 8)
    sizes = list(wl.sizes)
    k = [oracle_k(s, wl.densities[0]) for s in sizes]
    run(sizes, [k] * 3, lambda w, s: W.gradient(wl, w, s), wl.clip, path=path, grid=grid,
        tag=f"rn50/8 p{path} g{grid}")


def test_warmup_schedule_scaled():
    """One 3.5M tensor through the warm-up densities 1/4 ... 1/1000."""
    wl = W.scaled(W.get("warmup350m"), 100)
    n = wl.n
    ks = [[oracle_k(n, d)] for d in wl.densities]
    for grid in (0, 2):
        run([n], ks, lambda w, s: W.gradient(wl, w, s), wl.clip, grid=grid,
            tag=f"warm/100 g{grid}")


@pytest.mark.parametrize("grid", [0, 1, 2])
def test_long_tensor_layout(grid):
    """A tensor above 2**22 elements keeps the layout on the spread path;
    grid 1 then takes the per-tensor select."""
    rng = np.random.default_rng(81)
    sizes = [(1 << 22) + 5, 70001, 300, 0, 33]
    n = sum(sizes)
    k = [oracle_k(s, Fraction(1, 1000)) for s in sizes]
    grads = [rng.laplace(0, 1e-3, n).astype(np.float32) for _ in range(2)]
    run(sizes, [k, k], lambda w, s: grads[s], 0.5, grid=grid, tag=f"long g{grid}")


def test_flat1b_shape_scaled_four_learners():
    wl = W.scaled(W.get("flat1b"), 256)
    sizes = list(wl.sizes)
    k = [oracle_k(s, wl.densities[0]) for s in sizes]
    run(sizes, [k] * 2, lambda w, s: W.gradient(wl, w, s), wl.clip, learners=4, tag="1b/256")


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts(seed):
    """1-30 tensors of 0 to 300k elements around the whole-sample limit, k
    from 0 to n, sparse or dense gradients, clipping on or off, all paths."""
    rng = np.random.default_rng([82, seed])
    T = int(rng.integers(1, 31))
    sizes = [int(x) for x in rng.choice([0, 1, 7, 32, 33, 1000, 65535, 65536, 65537,
                                         131075, 299999], T)]
    n = sum(sizes)
    ks = []
    for _ in range(2):
        ks.append([int(rng.integers(0, s + 1)) if rng.random() < 0.3 else -(-s // 100)
                   for s in sizes])
    grads = []
    for _ in range(2):
        g = rng.laplace(0, 1e-2, n).astype(np.float32)
        g[rng.random(n) < rng.choice([0.05, 0.995])] = 0.0
        grads.append(g)
    clip = float(rng.choice([0.0, 0.5]))
    for path, grid in GRIDS:
        run(sizes, ks, lambda w, s: grads[s], clip, path=path, grid=grid,
            tag=f"fuzz{seed} p{path} g{grid}")


def segments(n, segs):
    g = np.zeros(n, np.float32)
    for a, b, x in segs:
        g[a:b] = x
    return g


@pytest.mark.parametrize("path,grid", GRIDS)
def test_hand_derived_cases(path, grid):
    """The oracle's hand-derived cases (tests/golden/hier_cases.json) as
    tensors of one layout: an overshoot, an undershoot (theta 0: only the
    non-zero entries survive), exactly k, ties across a gap and k = 0."""
    from conftest import load_golden
    c = load_golden("hier_cases.json")
    n = c["n"]
    cases = c["cases"]
    g = np.concatenate([segments(n, cs["segments"]) for cs in cases])
    k = [cs["k"] for cs in cases]
    sizes = [n] * len(cases)
    pair = HierPair(sizes, [max(x, 1) for x in k], path=path, grid=grid)
    say(f"hand cases p{path} g{grid}")
    _, _, o_cnt = pair.step(g, k, 0.0, tag=f"hand p{path} g{grid}")
    assert o_cnt.tolist() == [cs["count"] for cs in cases]


@pytest.mark.parametrize("grid", [0, 2])
def test_overflowing_pieces_take_the_whole_tensor(grid):
    """500 large entries in one 1024-element piece overflow its slots
    (k_max = 1000 gives 30 per piece): that tensor's select runs on the
    whole tensor under the floor; with many zeros the survivors fall short
    of k and T is 0 there."""
    rng = np.random.default_rng(83)
    n = 1 << 20
    def grads(w, s):
        g = rng.laplace(0, 1e-3, 2 * n).astype(np.float32)  # two tensors of n
        for o in (0, n):
            g[o + 4096:o + 4096 + 500] = rng.choice([-1.0, 1.0], 500) * rng.uniform(1, 2, 500)
        if s == 1:
            g[rng.random(2 * n) < 0.999] = 0.0
            g[8192:8192 + 400] = 3.0
        return g.astype(np.float32)
    seen = run([n, n], [[1000, 1000], [1000, 1000]], grads, 0.0, grid=grid,
               k_max=[1000, 1000], tag=f"overflow g{grid}")
    assert ("dense",) in seen, seen


def test_every_source_kind_is_exercised():
    """Over the layouts above the three kinds occur: a whole list of at most
    k survivors, a longer list selected from, and the whole tensor."""
    wl = W.scaled(W.get("resnet50"), 8)
    sizes = list(wl.sizes)
    k = [oracle_k(s, wl.densities[0]) for s in sizes]
    seen = run(sizes, [k] * 2, lambda w, s: W.gradient(wl, w, s), wl.clip, tag="kinds")
    assert ("list", "whole") in seen and ("list", "select") in seen, seen
    seen = run(sizes, [k], lambda w, s: W.gradient(wl, w, s), wl.clip, path=1,
               tag="kinds dense")
    assert seen == {("dense",)}, seen


def test_all_k_zero_writes_zero_counts():
    """Both the per-tensor kernels and the spread passes write E_t = 0."""
    import torch
    for sizes in ([1000, 5000], [1000, (1 << 22) + 1]):
        for grid in (0, 2):
            L = dgc.Learner(sizes, [10, 10])
            L.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
            L.count.fill_(7)
            g = torch.ones(sum(sizes), device="cuda")
            _, _, count = L.compress_hier(g, [0, 0], 0.0)
            torch.cuda.synchronize()
            assert count.cpu().tolist() == [0, 0], (sizes, grid)
            assert L.status() == dgc.DGC_OK
            L.close()


def test_bad_arguments():
    import torch
    L = dgc.Learner([1000, 5000], [1000, 100])
    g = torch.zeros(6000, device="cuda")
    for k in ([1001, 1], [-1, 1], [5, 101]):
        with pytest.raises(dgc.DGCError) as e:
            L.compress_hier(g, k, 0.0)
        assert e.value.code == dgc.DGC_EINVAL
    with pytest.raises(dgc.DGCError):
        dgc.dgc_compress_hier(L.state, g, [1, 1], 0.0, L.idx, L.val, None)
    # a gradient shorter than the layout is refused before any launch
    with pytest.raises(ValueError):
        L.compress_hier(g[:5999], [1, 1], 0.0)
    with pytest.raises(ValueError):
        L.compress(g.double(), [1, 1], 0.0)
