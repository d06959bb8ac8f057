"""GPU parity of the sampled-threshold selector (DGC review, "Research
questions", RQ4): dgc_compress_sampled + dgc_encode_counts + decode through
the C ABI against the CPU oracle, bit for bit on the threshold, the delivered
and at-threshold counts, indices, values, u/v state, streams and dense sums.

Layouts mix whole-tensor samples (<= 65536 elements) and line samples, with
unaligned tensor starts and ragged tails; k from 0 to n; capacities from
none to all; both placement paths.
"""

import numpy as np
import pytest

import oracle
from gpu_harness import f32_bits, first_diff, oracle_k, say
from sparsified_gradient_compression_amd import dgc
from sparsified_gradient_compression_amd import workloads as W
from test_gpu_binlocal import check_decode

pytestmark = pytest.mark.gpu

SAMPLED_PATH = 3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dgc.lib()
    return torch


class SampledPair:
    def __init__(self, sizes, k_max, momentum=0.9, path=0):
        self.sizes = [int(s) for s in sizes]
        self.learner = dgc.Learner(self.sizes, k_max, momentum)
        self.learner.set_option(dgc.DGC_OPT_SELECT_PATH, path)
        n = sum(self.sizes)
        self.u = np.zeros(n, np.float32)
        self.v = np.zeros(n, np.float32)
        self.m = momentum

    def step(self, g, k, cap, clip, tag=""):
        import torch
        lr = self.learner
        idx, val, count, total = lr.compress_sampled(torch.from_numpy(g).cuda(), k, cap, clip)
        torch.cuda.synchronize()
        g_idx = idx.cpu().numpy().view(np.uint32)
        g_val = val.cpu().numpy()
        g_cnt = count.cpu().numpy()
        g_tot = total.cpu().numpy()
        info = lr.select_info()
        o_idx, o_val, o_cnt, o_tot, o_th, o_norm, o_s = oracle.sampled_step(
            self.sizes, k, cap, g, self.u, self.v, self.m, clip)
        assert lr.status() == dgc.DGC_OK, (tag, "status")
        assert (info[:, 0] == SAMPLED_PATH).all(), (tag, info[:, 0])
        th = info[:, 4].astype(np.uint32)
        assert np.array_equal(th, o_th), (tag, "theta", first_diff(th, o_th))
        assert np.array_equal(g_tot, o_tot), (tag, "total", first_diff(g_tot, o_tot))
        assert np.array_equal(g_cnt, o_cnt), (tag, "count", first_diff(g_cnt, o_cnt))
        if clip > 0:
            norm = float(lr.norm.cpu()[0])
            assert abs(norm - o_norm) <= 1e-6 * o_norm, (tag, norm, o_norm)
        assert np.float32(lr.scale.cpu()[0]) == o_s, (tag, "scale")
        off = 0
        for t, c in enumerate(cap):
            a, b = off, off + int(o_cnt[t])
            assert np.array_equal(g_idx[a:b], o_idx[a:b]), (tag, t, "idx",
                                                            first_diff(g_idx[a:b], o_idx[a:b]))
            assert np.array_equal(f32_bits(g_val[a:b]), f32_bits(o_val[a:b])), (tag, t, "val")
            off += int(c)
        gu = lr.u[: len(self.u)].cpu().numpy()
        gv = lr.v[: len(self.v)].cpu().numpy()
        assert np.array_equal(f32_bits(gu), f32_bits(self.u)), (
            tag, "u", first_diff(f32_bits(gu), f32_bits(self.u)))
        assert np.array_equal(f32_bits(gv), f32_bits(self.v)), (
            tag, "v", first_diff(f32_bits(gv), f32_bits(self.v)))
        return o_idx, o_val, o_cnt, o_tot

    def check_encode(self, cap, o_idx, o_val, o_cnt, tag=""):
        import torch
        runs, vals, entries = self.learner.encode_counts(cap)
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
                                   cap=max(int(cap[t]) + nt // 65536, 1))
            assert np.array_equal(r[scap[t]:scap[t] + e[t]], wr), (tag, t, "runs")
            assert np.array_equal(f32_bits(v[scap[t]:scap[t] + e[t]]), f32_bits(wv)), (tag, t)
            want.append((wr, wv))
            off += int(cap[t])
        return want


def run(sizes, ks, caps, grads, clip, learners=1, path=0, k_max=None, tag=""):
    """ks[step], caps[step]: per-tensor lists; grads(w, step) -> float32[n]."""
    k_max = list(sizes) if k_max is None else k_max
    pairs = [SampledPair(sizes, k_max, path=path) for _ in range(learners)]
    for step, (k, cap) in enumerate(zip(ks, caps)):
        streams = []
        for w, p in enumerate(pairs):
            say(f"{tag} step {step} learner {w} T={len(sizes)} n={sum(sizes)}")
            o_idx, o_val, o_cnt, _ = p.step(grads(w, step), k, cap, clip,
                                            tag=f"{tag} s{step} w{w}")
            streams.append(p.check_encode(cap, o_idx, o_val, o_cnt, tag=f"{tag} s{step} w{w}"))
        check_decode(pairs, streams, sizes, tag=f"{tag} s{step}")
    return pairs


@pytest.mark.parametrize("path", [0, 1])
def test_flat1m(path):
    wl = W.get("flat1m")
    n = wl.n
    k = [oracle_k(n, wl.densities[0])]
    run([n], [k, k], [[n], [n]], lambda w, s: W.gradient(wl, w, s), 0.0, path=path,
        tag=f"flat1m p{path}")


@pytest.mark.parametrize("path", [0, 1])
def test_resnet50_layout_scaled(path):
    """161 tensors scaled 1/8: most are whole-tensor samples, the largest
    are line samples; k = ceil(n/1000), clipping on, three steps."""
    wl = W.scaled(W.get("resnet50"), 8)
    sizes = list(wl.sizes)
    k = [oracle_k(s, wl.densities[0]) for s in sizes]
    cap = [min(s, 4 * kk + 64) for s, kk in zip(sizes, k)]
    run(sizes, [k] * 3, [cap] * 3, lambda w, s: W.gradient(wl, w, s), wl.clip,
        k_max=cap, path=path, tag=f"rn50/8 p{path}")


def test_warmup_schedule_scaled():
    """One 3.5M tensor through the warm-up densities 1/4 ... 1/1000."""
    wl = W.scaled(W.get("warmup350m"), 100)
    n = wl.n
    ks = [[oracle_k(n, d)] for d in wl.densities]
    run([n], ks, [[n]] * len(ks), lambda w, s: W.gradient(wl, w, s), wl.clip, tag="warm/100")


def test_flat1b_shape_scaled_four_learners():
    wl = W.scaled(W.get("flat1b"), 256)
    sizes = list(wl.sizes)
    k = [oracle_k(s, wl.densities[0]) for s in sizes]
    cap = [4 * kk for kk in k]
    run(sizes, [k] * 2, [cap] * 2, lambda w, s: W.gradient(wl, w, s), wl.clip, learners=4,
        k_max=cap, tag="1b/256")


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts(seed):
    """1-30 tensors of 0 to 300k elements around the whole-sample limit, k
    from 0 to n, capacities from 0 to n, clipping on or off, both paths."""
    rng = np.random.default_rng([71, seed])
    T = int(rng.integers(1, 31))
    sizes = [int(x) for x in rng.choice([0, 1, 7, 32, 33, 1000, 65535, 65536, 65537,
                                         131075, 299999], T)]
    n = sum(sizes)
    ks, caps = [], []
    for _ in range(2):
        ks.append([int(rng.integers(0, s + 1)) if rng.random() < 0.3 else -(-s // 100)
                   for s in sizes])
        caps.append([s if rng.random() < 0.5 else int(rng.integers(0, s // 20 + 2))
                     for s in sizes])
    caps = [[min(c, s) for c, s in zip(cc, sizes)] for cc in caps]
    k_max = [max(caps[0][i], caps[1][i]) for i in range(T)]
    grads = []
    for _ in range(2):
        g = rng.laplace(0, 1e-2, n).astype(np.float32)
        g[rng.random(n) < 0.05] = 0.0
        grads.append(g)
    clip = float(rng.choice([0.0, 0.5]))
    for path in (0, 1):
        run(sizes, ks, caps, lambda w, s: grads[s], clip, path=path, k_max=k_max,
            tag=f"fuzz{seed} p{path}")


def test_ties_and_zeros():
    """Few distinct magnitudes: the threshold ties many entries (all sent)."""
    rng = np.random.default_rng(72)
    sizes = [70001, 4096, 300]
    n = sum(sizes)
    def grads(w, s):
        g = rng.choice(np.array([0.0, 1e-40, 0.125, 0.25, 0.5]), n)
        return (g * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    k = [700, 41, 3]
    run(sizes, [k] * 3, [sizes] * 3, grads, 0.0, tag="ties")


def test_bad_arguments():
    import torch
    L = dgc.Learner([1000, 5000], [1000, 100])
    g = torch.zeros(6000, device="cuda")
    for k, cap in (([1001, 1], [1, 1]), ([-1, 1], [1, 1]), ([5, 5], [1, 101])):
        with pytest.raises(dgc.DGCError) as e:
            L.compress_sampled(g, k, cap, 0.0)
        assert e.value.code == dgc.DGC_EINVAL
    # k above k_max is allowed (k_max bounds only the delivered entries)
    L.compress_sampled(g, [10, 5000], [10, 100], 0.0)
    import torch as _t
    _t.cuda.synchronize()
    assert L.status() == dgc.DGC_OK
    assert L.count.cpu().tolist() == [0, 0]  # all zero: nothing sent
