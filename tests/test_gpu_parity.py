"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for
bit on selected indices, values, encoded streams, u/v state and dense sums;
the clipping norm to relative 1e-6.

Sizes here span several pieces and tiles with ragged tails; the full-size
workloads are in test_gpu_fullsize.py.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from gpu_harness import (Pair, compare_streams, f32_bits, first_diff,
                         gpu_streams, oracle_k, oracle_streams, say)
from sparsified_gradient_compression_amd import dgc
from sparsified_gradient_compression_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dgc.lib()  # raises if the HIP library is missing
    return torch


def ks_for(wl, step):
    return [oracle_k(s, wl.densities[step]) for s in wl.sizes]


def run_workload(wl, steps=None, learners=None, path=0, grid=0, encode=True, tag=""):
    steps = wl.steps if steps is None else steps
    learners = wl.learners if learners is None else learners
    kmax = [max(oracle_k(s, d) for d in wl.densities) for s in wl.sizes]
    pairs = [Pair(list(wl.sizes), kmax, wl.momentum) for _ in range(learners)]
    for p in pairs:
        p.learner.set_option(dgc.DGC_OPT_SELECT_PATH, path)
        p.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
    for t in range(steps):
        k = ks_for(wl, t)
        outs = []
        for w, p in enumerate(pairs):
            say(f"{tag} step {t} learner {w} n={wl.n} T={len(wl.sizes)}")
            g = W.gradient(wl, w, t)
            got, (o_idx, o_val) = p.step(g, k, wl.clip, tag=f"{tag} s{t} w{w}")
            check_paths(p, wl.sizes, k, path, grid, tag=f"{tag} s{t} w{w}")
            if encode:
                want = oracle_streams(wl.sizes, k, o_idx, o_val)
                gs = gpu_streams(p, k)
                compare_streams(gs, want, tag=f"{tag} s{t} w{w}")
                outs.append(want)
        if encode:
            check_decode(pairs, outs, wl.sizes, tag=f"{tag} s{t}")
    return pairs


SMALL_N = 65536  # on the spread passes, tensors up to this size take the dense path
TENSOR_PATH_MAX_N = 1 << 22  # layouts within this take the per-tensor kernels


def check_paths(pair, sizes, k, path, grid=0, tag=""):
    """On unstructured gradients the automatic path takes the sample window
    for every tensor with k > 0 -- on the per-tensor kernels (every tensor
    at most 2^22 elements, grid not forced to the spread passes) small
    tensors too, since their whole tensor is sampled; on the spread passes
    only those above SMALL_N elements, the smaller ones taking the dense
    path.  The forced dense path is dense throughout."""
    per_tensor = grid != 2 and max(sizes) <= TENSOR_PATH_MAX_N
    info = pair.learner.select_info()
    for t, (n, kt) in enumerate(zip(sizes, k)):
        window = path == 0 and (n > SMALL_N or per_tensor)
        want = 0 if kt == 0 else (1 if window else 2)
        assert info[t, 0] == want, (tag, t, n, kt, info[t].tolist())


def check_decode(pairs, streams_per_learner, sizes, tag=""):
    """Decode every learner's GPU-encoded stream (learner order) into one
    dense sum and compare with the oracle decoding the oracle's streams:
    accumulated onto zeros (dgc_decode_accumulate) and as a fresh sum
    written over NaNs (dgc_decode_sum, what the benchmark times)."""
    import torch
    n = int(sum(sizes))
    want = np.zeros(n, np.float32)
    off = np.concatenate([[0], np.cumsum(sizes)])
    for streams in streams_per_learner:
        for t, (wr, wv) in enumerate(streams):
            assert oracle.decode_accumulate(wr, wv, want[off[t]:off[t + 1]]) == 0
    streams = [(p.learner.runs, p.learner.vals, p.learner.entries) for p in pairs]
    for fresh in (False, True):
        if fresh:
            dense = torch.full((max(n, 1),), float("nan"), dtype=torch.float32, device="cuda")
            dgc.decode_sum(pairs[0].learner, streams, dense)
        else:
            dense = torch.zeros(max(n, 1), dtype=torch.float32, device="cuda")
            dgc.decode_accumulate(pairs[0].learner, streams, dense)
        got = dense[:n].cpu().numpy()
        assert pairs[0].learner.status() == dgc.DGC_OK
        assert np.array_equal(f32_bits(got), f32_bits(want)), (tag, fresh, first_diff(got, want))
        del dense


# ---------------------------------------------------------------- workloads

# GRIDS: the exact select and emit as one workgroup per tensor (1) or as
# passes spread over the chip (2); the automatic choice takes 1 for every
# layout here, so both are forced.
GRIDS = [1, 2]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("path", [0, 1])
def test_flat1m(path, grid):
    """2**20 Laplace entries, k = 1049, one step, no clipping."""
    run_workload(W.get("flat1m"), path=path, grid=grid, tag=f"flat1m/p{path}g{grid}")


@pytest.mark.parametrize("grid", GRIDS)
def test_resnet50_scaled_three_steps(grid):
    wl = W.scaled(W.get("resnet50"), 8)
    run_workload(wl, steps=3, grid=grid, tag=f"rn50/8 g{grid}")


@pytest.mark.parametrize("grid", GRIDS)
def test_deepspeech_scaled_four_learners(grid):
    wl = W.scaled(W.get("deepspeech"), 40)
    run_workload(wl, grid=grid, tag=f"ds/40 g{grid}")


@pytest.mark.parametrize("grid", GRIDS)
def test_warmup_schedule_scaled(grid):
    wl = W.scaled(W.get("warmup350m"), 100)
    run_workload(wl, grid=grid, tag=f"warm/100 g{grid}")


def test_flat1b_shape_scaled():
    wl = W.scaled(W.get("flat1b"), 256)
    run_workload(wl, steps=2, learners=2, tag="1b/256")


# ---------------------------------------------------------------- edge cases

RAGGED = [1, 0, 3, 64, 1000, 1023, 1025, 4097, 65536, 65537, 300001, 7]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("seed", [0, 1])
def test_ragged_layout(path, seed, grid):
    """Odd sizes (misaligned tensor starts, partial float4 units, partial
    pieces and tiles), an empty tensor, k from 0 to n."""
    rng = np.random.default_rng([31, seed])
    sizes = list(RAGGED)
    n = sum(sizes)
    ks_steps = []
    for step in range(3):
        k = []
        for s in sizes:
            choice = rng.integers(0, 5)
            k.append([0, 1, s, max(1, s // 1000) if s else 0,
                      int(rng.integers(0, s + 1))][choice] if s else 0)
        ks_steps.append(k)
    kmax = [max(ks[t] for ks in ks_steps) for t in range(len(sizes))]
    p = Pair(sizes, kmax)
    p.learner.set_option(dgc.DGC_OPT_SELECT_PATH, path)
    p.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
    for step, k in enumerate(ks_steps):
        g = (rng.laplace(0, 1e-2, n) * (rng.random(n) < 0.9)).astype(np.float32)
        clip = [0.0, 0.5, 1e6][step]
        got, (o_idx, o_val) = p.step(g, k, clip, tag=f"ragged s{step}")
        want = oracle_streams(sizes, k, o_idx, o_val)
        compare_streams(gpu_streams(p, k), want, tag=f"ragged s{step}")
        check_decode([p], [want], sizes, tag=f"ragged s{step}")


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("path", [0, 1])
def test_ties_and_zeros(path, grid):
    """Few distinct magnitudes (ties at the threshold everywhere), signed
    zeros, an all-zero tensor, and k = n."""
    rng = np.random.default_rng(32)
    sizes = [200000, 70000, 5000, 131072]
    n = sum(sizes)
    pool = np.array([0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 0.25], np.float32)
    p = Pair(sizes, sizes)
    p.learner.set_option(dgc.DGC_OPT_SELECT_PATH, path)
    p.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
    for step, k in enumerate([[200, 70, 5000, 131], [199999, 0, 1, 131072],
                              [1, 69999, 2500, 65536]]):
        g = pool[rng.integers(0, pool.size, n)]
        g[200000:270000] = 0.0 if step != 1 else -0.0
        got, (o_idx, o_val) = p.step(g, k, 0.0, tag=f"ties s{step}")
        compare_streams(gpu_streams(p, k), oracle_streams(sizes, k, o_idx, o_val),
                        tag=f"ties s{step}")


def test_both_paths_agree_and_window_is_used():
    wl = W.scaled(W.get("flat1b"), 64)
    k = ks_for(wl, 0)
    g = W.gradient(wl, 0, 0)
    res = []
    for path in (0, 1):
        p = Pair(list(wl.sizes), k)
        p.learner.set_option(dgc.DGC_OPT_SELECT_PATH, path)
        got, _ = p.step(g, k, wl.clip, tag=f"paths p{path}")
        nw, nd = p.learner.path_counts()
        if path == 0:
            assert nd == 0 and nw == len(wl.sizes), (nw, nd)
        else:
            assert nw == 0 and nd == len(wl.sizes), (nw, nd)
        res.append(got)
    assert np.array_equal(res[0].idx, res[1].idx)


def test_determinism_repeat_bitwise():
    wl = W.scaled(W.get("resnet50"), 16)
    outs = []
    for rep in range(2):
        p = Pair(list(wl.sizes), ks_for(wl, 0))
        for t in range(2):
            got, _ = p.step(W.gradient(wl, 0, t), ks_for(wl, t), wl.clip,
                            check_state=False, tag=f"det r{rep}")
        outs.append((got.idx, f32_bits(got.val), p.learner.v.cpu().numpy().copy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(f32_bits(outs[0][2]), f32_bits(outs[1][2]))


def test_checkpoint_resume_bitwise():
    """The whole learner state is (u, v): 4 steps straight equal 2 steps,
    a save/restore of u and v into a fresh state, then 2 more steps."""
    import torch
    wl = W.scaled(W.get("resnet50"), 32)
    wl = W.Workload(wl.name, wl.cfg_id, wl.sizes, (Fraction(1, 1000),) * 4, 1,
                    wl.clip, wl.momentum, wl.dist)
    k = ks_for(wl, 0)
    a = Pair(list(wl.sizes), k)
    for t in range(4):
        ga, _ = a.step(W.gradient(wl, 0, t), k, wl.clip, tag=f"ckpt a{t}")
    b = Pair(list(wl.sizes), k)
    for t in range(2):
        b.step(W.gradient(wl, 0, t), k, wl.clip, tag=f"ckpt b{t}")
    saved_u = b.learner.u.clone()
    saved_v = b.learner.v.clone()
    c = Pair(list(wl.sizes), k)
    c.learner.u.copy_(saved_u)
    c.learner.v.copy_(saved_v)
    c.u, c.v = b.u.copy(), b.v.copy()
    for t in range(2, 4):
        gc, _ = c.step(W.gradient(wl, 0, t), k, wl.clip, tag=f"ckpt c{t}")
    assert np.array_equal(ga.idx, gc.idx)
    assert torch.equal(a.learner.v, c.learner.v)


# ---------------------------------------------------------------- codec

ENCODE_PATHS = [1, 2]  # DGC_OPT_ENCODE_PATH: a workgroup per tensor; the tiled passes


@pytest.mark.parametrize("enc", ENCODE_PATHS)
def test_encode_golden_gaps_on_gpu(enc):
    """The hand-derived streams of tests/golden/encode_cases.json, encoded
    by the GPU from the golden indices, on both encode paths."""
    import torch
    from conftest import load_golden
    gold = load_golden("encode_cases.json")
    for case in gold["cases"]:
        n = case["n"]
        idx = np.array(case["idx"], np.uint32)
        val = np.array([int(h, 16) for h in case["val"]], np.uint32).view(np.float32)
        k = [idx.size]
        p = Pair([n], [max(idx.size, 1)])
        ti = torch.from_numpy(idx.view(np.int32)).cuda()
        tv = torch.from_numpy(val).cuda()
        L = p.learner
        L.set_option(dgc.DGC_OPT_ENCODE_PATH, enc)
        L.idx[:idx.size].copy_(ti)
        L.val[:idx.size].copy_(tv)
        got = gpu_streams(p, k)[0]
        want = oracle.encode(idx, val, cap=idx.size + n // 65536 + 1)
        assert np.array_equal(got[0], want[0]), case["name"]
        assert np.array_equal(f32_bits(got[1]), f32_bits(want[1])), case["name"]
        runs_w = case.get("runs")
        if runs_w is None:
            runs_w = sum(([x] * c for x, c in case["runs_repeat"]), [])
        assert got[0].tolist() == runs_w, case["name"]
        assert L.status() == dgc.DGC_OK


def test_decode_flags_corrupt_streams():
    import torch
    sizes = [10, 100000]
    p = Pair(sizes, [3, 5])
    L = p.learner
    cap = L.cap
    runs = torch.zeros(int(cap[-1]), dtype=torch.int16, device="cuda")
    vals = torch.ones(int(cap[-1]), dtype=torch.float32, device="cuda")
    # tensor 0: positions 3, 8, 14 -> the third passes the end (n = 10)
    runs[0:3] = torch.tensor([3, 4, 5], dtype=torch.int16)
    ent = torch.tensor([3, 0], dtype=torch.int64, device="cuda")
    dense = torch.zeros(sum(sizes), dtype=torch.float32, device="cuda")
    dgc.decode_accumulate(L, [(runs, vals, ent)], dense)
    assert L.status() == dgc.DGC_ECORRUPT
    assert L.status() == dgc.DGC_OK  # cleared by the read
    d = dense.cpu().numpy()
    assert d[3] == 1 and d[8] == 1 and d.sum() == 2
    # an entry count above capacity adds nothing and is flagged
    ent2 = torch.tensor([int(cap[1] - cap[0]) + 1, 0], dtype=torch.int64, device="cuda")
    dense.zero_()
    dgc.decode_accumulate(L, [(runs, vals, ent2)], dense)
    assert L.status() == dgc.DGC_ECORRUPT
    assert float(dense.abs().sum()) == 0.0


def test_k_above_k_max_is_rejected():
    import torch
    p = Pair([1000], [5])
    g = torch.zeros(1000, device="cuda")
    with pytest.raises(dgc.DGCError):
        p.learner.compress(g, [6], 0.0)
    g1 = torch.zeros(1001, device="cuda")
    with pytest.raises(dgc.DGCError):
        p.learner.compress(g1[1:], [1], 0.0)  # misaligned gradient (1000 elements)


def test_pipelined_learners_on_streams():
    """Four learners on four streams, each starting once the previous one's
    element-wise pass is done (the library records the caller's event after
    it); encode on the learner's stream, decode on the main stream.  Every
    learner's outputs and state, and the dense sum, equal the oracle's."""
    import torch
    wl = W.scaled(W.get("flat1b"), 64)
    k = ks_for(wl, 0)
    sizes = np.array(wl.sizes, np.int64)
    pairs = [Pair(list(wl.sizes), k, wl.momentum) for _ in range(wl.learners)]
    streams = [torch.cuda.Stream() for _ in pairs]
    events = [torch.cuda.Event() for _ in pairs]
    for p, ev in zip(pairs, events):
        p.learner.set_fused_event(ev)
    main = torch.cuda.current_stream()
    n = wl.n
    dense = torch.zeros(n, dtype=torch.float32, device="cuda")
    for t in range(2):
        grads = [W.gradient(wl, w, t) for w in range(wl.learners)]
        dev = [torch.from_numpy(g).cuda() for g in grads]
        torch.cuda.synchronize()
        for w, p in enumerate(pairs):
            st = streams[w]
            if w == 0:
                st.wait_stream(main)
            else:
                st.wait_event(events[w - 1])
            with torch.cuda.stream(st):
                p.learner.compress(dev[w], k, wl.clip, stream=st)
                p.learner.encode(k, stream=st)
        for st in streams:
            main.wait_stream(st)
        dense.zero_()
        dgc.decode_accumulate(pairs[0].learner,
                              [(p.learner.runs, p.learner.vals, p.learner.entries)
                               for p in pairs], dense)
        torch.cuda.synchronize()
        want_dense = np.zeros(n, np.float32)
        offs = np.concatenate([[0], np.cumsum(sizes)])
        koff = np.concatenate([[0], np.cumsum(k)])
        for w, p in enumerate(pairs):
            o_idx, o_val, o_norm, o_s = oracle.step(sizes, np.array(k), grads[w], p.u, p.v,
                                                    wl.momentum, wl.clip)
            L = p.learner
            assert L.status() == dgc.DGC_OK
            assert np.array_equal(L.idx[:o_idx.size].cpu().numpy().view(np.uint32), o_idx)
            assert np.array_equal(f32_bits(L.val[:o_val.size].cpu().numpy()), f32_bits(o_val))
            assert np.array_equal(f32_bits(L.u[:n].cpu().numpy()), f32_bits(p.u))
            assert np.array_equal(f32_bits(L.v[:n].cpu().numpy()), f32_bits(p.v))
            for tt in range(len(k)):
                r, vv = oracle.encode(o_idx[koff[tt]:koff[tt + 1]], o_val[koff[tt]:koff[tt + 1]])
                assert oracle.decode_accumulate(r, vv, want_dense[offs[tt]:offs[tt + 1]]) == 0
        assert np.array_equal(f32_bits(dense.cpu().numpy()), f32_bits(want_dense))
    for p in pairs:
        p.learner.set_fused_event(None)


def _keys(v):
    return np.asarray(v, np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts_both_paths(seed):
    """Seeded random layouts: 1-40 tensors of 1 to 400k elements (odd sizes,
    so tensor starts are misaligned), random k per step, clipping on or
    off, Laplace gradients with zero runs; both selection paths must give
    the oracle's bits.  The per-tensor threshold key T and tie quota r the
    library reports must equal the oracle's: T = the k-th largest key of the
    accumulated v, r = k - #{key > T}."""
    rng = np.random.default_rng([41, seed])
    T = int(rng.integers(1, 41))
    sizes = [int(x) for x in rng.choice([1, 2, 7, 300, 1023, 4099, 65535, 65537,
                                         131075, 399999], T)]
    n = sum(sizes)
    steps = 2
    ks = [[int(rng.integers(0, s + 1)) if rng.random() < 0.3 else -(-s // 1000)
           for s in sizes] for _ in range(steps)]
    kmax = [max(ks[t][i] for t in range(steps)) for i in range(T)]
    for path, grid in ((0, 1), (0, 2), (1, 1), (1, 2)):
        p = Pair(sizes, kmax)
        p.learner.set_option(dgc.DGC_OPT_SELECT_PATH, path)
        p.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
        for step in range(steps):
            g = rng.laplace(0, 1e-2, n).astype(np.float32)
            g[rng.random(n) < 0.05] = 0.0
            clip = float(rng.choice([0.0, 0.5, 100.0]))
            u0, v0 = p.u.copy(), p.v.copy()
            got, (o_idx, o_val) = p.step(g, ks[step], clip, tag=f"fuzz{seed} p{path}g{grid} s{step}")
            # the accumulated v before masking, from the oracle's own steps
            _, s32 = oracle.clip_scale(g, clip)
            oracle.momentum(g, s32, 0.9, u0, v0)
            info = p.learner.select_info()
            off = np.concatenate([[0], np.cumsum(sizes)])
            for t in range(T):
                k_t = ks[step][t]
                if k_t == 0:
                    assert info[t, 0] == 0
                    continue
                keys = _keys(v0[off[t]:off[t + 1]])
                Tk = np.sort(keys)[::-1][k_t - 1]
                r = k_t - int((keys > Tk).sum())
                assert info[t, 4] == Tk and info[t, 5] == r, (seed, path, step, t,
                                                              info[t].tolist(), int(Tk), r)
            want = oracle_streams(sizes, ks[step], o_idx, o_val)
            compare_streams(gpu_streams(p, ks[step]), want, tag=f"fuzz{seed}")


@pytest.mark.parametrize("enc", ENCODE_PATHS)
def test_encode_flags_unsorted_indices(enc):
    """dgc_encode expects each tensor's indices strictly ascending and inside
    the tensor; anything else latches DGC_ECORRUPT and writes nothing out of
    place."""
    import torch
    p = Pair([1000, 70000], [4, 4])
    L = p.learner
    L.set_option(dgc.DGC_OPT_ENCODE_PATH, enc)
    bad = np.array([5, 3, 9, 12, 1, 2, 70000, 7], np.uint32)  # descending / out of range
    L.idx[:8].copy_(torch.from_numpy(bad.view(np.int32)))
    L.val[:8].copy_(torch.ones(8))
    L.runs.zero_()
    L.encode([4, 4])
    torch.cuda.synchronize()
    assert L.status() == dgc.DGC_ECORRUPT
    assert L.status() == dgc.DGC_OK
    assert int(L.runs.abs().max()) <= 65535


def test_kernel_timers():
    import torch
    wl = W.scaled(W.get("flat1b"), 64)
    k = ks_for(wl, 0)
    p = Pair(list(wl.sizes), k)
    L = p.learner
    L.set_option(dgc.DGC_OPT_KERNEL_TIMING, 1)
    g = torch.from_numpy(W.gradient(wl, 0, 0)).cuda()
    for _ in range(3):
        L.compress(g, k, wl.clip)
        L.encode(k)
    ms_f, n_f = L.kernel_time(dgc.DGC_TIMER_FUSED)
    ms_c, n_c = L.kernel_time(dgc.DGC_TIMER_COMPRESS)
    ms_e, n_e = L.kernel_time(dgc.DGC_TIMER_ENCODE)
    assert (n_f, n_c, n_e) == (3, 3, 3)
    assert 0 < ms_f < ms_c and ms_e > 0
    assert L.kernel_time(dgc.DGC_TIMER_FUSED) == (0.0, 0)  # read resets
    # mode 2: the element-wise pass only; mode 3: each call but not that pass
    for mode, want in ((2, (2, 0, 0)), (3, (0, 2, 2))):
        L.set_option(dgc.DGC_OPT_KERNEL_TIMING, mode)
        for _ in range(2):
            L.compress(g, k, wl.clip)
            L.encode(k)
        got = tuple(L.kernel_time(t)[1] for t in (dgc.DGC_TIMER_FUSED, dgc.DGC_TIMER_COMPRESS,
                                                 dgc.DGC_TIMER_ENCODE))
        assert got == want, (mode, got)
    with pytest.raises(dgc.DGCError):
        L.set_option(dgc.DGC_OPT_KERNEL_TIMING, 4)
    L.set_option(dgc.DGC_OPT_KERNEL_TIMING, 0)


def test_empty_layout():
    """Every tensor empty: compress, encode and decode do nothing and report
    norm -1 / scale 1 with clipping off (norm 0 / scale 1 with it on)."""
    import torch
    p = Pair([0, 0], [0, 0])
    L = p.learner
    g = torch.zeros(4, device="cuda")
    L.compress(g, [0, 0], 0.0)
    torch.cuda.synchronize()
    assert float(L.norm.cpu()[0]) == -1.0 and float(L.scale.cpu()[0]) == 1.0
    L.compress(g, [0, 0], 0.5)
    torch.cuda.synchronize()
    assert float(L.norm.cpu()[0]) == 0.0 and float(L.scale.cpu()[0]) == 1.0
    runs, vals, ent = L.encode([0, 0])
    torch.cuda.synchronize()
    assert ent.cpu().tolist() == [0, 0]
    dense = torch.zeros(4, device="cuda")
    dgc.decode_accumulate(L, [(runs, vals, ent)], dense)
    assert L.status() == dgc.DGC_OK


@pytest.mark.parametrize("grid", GRIDS)
def test_threshold_bin_crowded(grid):
    """T inside a cluster of keys that share their top 21 bits (values 1.0 +
    i ulp, i < 1000, each three times): on the per-tensor kernels the keys of
    T's 21-bit bin are too many (> 1024) to count one by one, so the last
    digit pass decides T and r; a candidate list that fits in LDS (3100
    items), one in memory (12100 items, above the 10240 that fit), and a
    short list (at most 128 candidates, selected by counting) with ties at
    T, against the oracle bit for bit."""
    rng = np.random.default_rng(77)
    sizes = [100000, 300000, 20000]
    n = sum(sizes)
    g = np.zeros(n, np.float32)
    one = np.float32(1.0).view(np.uint32)

    def cluster(lo, size, count, above):
        pos = lo + rng.permutation(size)[:count + above]
        ulps = np.arange(count) % 1000
        g[pos[:count]] = (one + ulps.astype(np.uint32)).view(np.float32)
        g[pos[:count]] *= rng.choice(np.float32([-1, 1]), count)
        g[pos[count:]] = np.float32(2.0)

    cluster(0, 100000, 3000, 100)
    cluster(100000, 300000, 12000, 100)
    # the short list: 100 keys at 0.5 and 20 at 0.75, k = 40 (20 ties sent)
    pos = 400000 + rng.permutation(20000)[:120]
    g[pos[:100]] = 0.5
    g[pos[100:]] = 0.75
    k = [1200, 4000, 40]
    p = Pair(sizes, k)
    p.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
    got, (o_idx, o_val) = p.step(g, k, 0.0, tag=f"crowded g{grid}")
    compare_streams(gpu_streams(p, k), oracle_streams(sizes, k, o_idx, o_val),
                    tag=f"crowded g{grid}")
    info = p.learner.select_info()
    # the spread passes take tensors of at most 65536 elements densely
    assert info[:, 0].tolist() == ([1, 1, 1] if grid == 1 else [1, 1, 2]), info.tolist()
    assert info[0, 2] == 3100 and info[1, 2] == 12100, info.tolist()
    if grid == 1:
        assert info[2, 2] == 120, info.tolist()
    assert info[2, 4] == np.float32(0.5).view(np.uint32) and info[2, 5] == 20, info.tolist()


@pytest.mark.parametrize("grid", GRIDS)
def test_dense_fallback_after_masking(grid):
    """The element-wise pass stores the window's candidates as +0 in every
    piece whose run fits its slots.  A tensor whose candidates then turn out
    incomplete takes the dense path, and those candidates must get their u
    and v back before the dense select reads v.  Tensor 0: one piece of
    large values (more candidates than its slots hold).  Tensor 1: 1% of
    entries tie at one large magnitude, about 10 per piece (every piece
    fits) but more than the candidate list holds.  Tensor 2: ordinary data
    on the list path.  Same bits as the oracle over two steps, the second on
    ordinary data added to the first step's residual."""
    rng = np.random.default_rng(77)
    sizes = [1 << 20, 1 << 22, 300000]
    k = [1000, 1000, 300]
    p = Pair(sizes, k)
    p.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    big = slice(5 * 1024, 6 * 1024)
    g[big] = rng.uniform(1.0, 2.0, 1024).astype(np.float32) * sign[big]
    t1 = slice(int(off[1]), int(off[2]))
    tie = rng.random(sizes[1]) < 0.01
    g1 = g[t1]
    g1[tie] = 0.5 * sign[t1][tie]
    p.step(g, k, 0.0, tag="fallback s0")
    info = p.learner.select_info()
    no_window = 0xFFFFFFFF
    # tensor 0: window used, a piece overflowed, dense path
    assert info[0, 1] != no_window and info[0, 3] == 1 and info[0, 0] == 2, info[0].tolist()
    # tensor 1: window used, no piece overflowed, too many candidates: dense
    assert info[1, 1] != no_window and info[1, 3] == 0 and info[1, 0] == 2, info[1].tolist()
    assert info[1, 2] > 8 * k[1] + 16384, info[1].tolist()
    assert info[2, 0] == 1, info[2].tolist()
    # the residual ties keep tensor 1 on the dense path; state and outputs
    # must still match
    p.step(rng.laplace(0, 1e-3, n).astype(np.float32), k, 0.0, tag="fallback s1")


@pytest.mark.parametrize("grid", [0, 2])
def test_dense_fallback_with_run_gather(grid):
    """At an average density of 1/8 or more the spread path's gather copies
    whole runs (several workgroups per piece group).  Tensors 0 and 2 (the
    last above 2^22 elements, so the layout takes the spread passes) select
    at density 1/4 from their lists; tensor 1 (k = 1000, about 29 slots per
    piece) has one piece of 500 large values that overflows, so it takes the
    dense path and the run gather must give its other pieces' candidates
    their u and v back.  Same bits as the oracle over two steps."""
    rng = np.random.default_rng(78)
    sizes = [1 << 20, 1 << 20, (1 << 22) + 3]
    k = [1 << 18, 1000, oracle_k(sizes[2], Fraction(1, 4))]
    assert sum(k) * 8 >= sum(sizes)
    p = Pair(sizes, k)
    p.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    a = int(off[1]) + 7 * 1024
    g[a:a + 500] = rng.uniform(1.0, 2.0, 500).astype(np.float32)
    p.step(g, k, 0.0, tag="run gather s0")
    info = p.learner.select_info()
    assert info[0, 0] == 1 and info[2, 0] == 1, info.tolist()
    assert info[1, 0] == 2 and info[1, 3] == 1, info[1].tolist()
    p.step(rng.laplace(0, 1e-3, n).astype(np.float32), k, 0.5, tag="run gather s1")


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("path", [0, 1])
def test_denormals_and_extremes(path, grid):
    """Denormal and near-overflow magnitudes: keys are bit patterns, so the
    order is exact and denormals are kept (no flush to zero)."""
    rng = np.random.default_rng(51)
    sizes = [100000, 3000, 262144]
    n = sum(sizes)
    p = Pair(sizes, [100, 3000, 262])
    p.learner.set_option(dgc.DGC_OPT_SELECT_PATH, path)
    p.learner.set_option(dgc.DGC_OPT_SELECT_GRID, grid)
    for step in range(2):
        g = rng.laplace(0, 1e-38, n).astype(np.float32)  # mostly denormal
        g[rng.random(n) < 0.001] = np.float32(1e38) * np.float32(rng.choice([-1, 1]))
        g[rng.random(n) < 0.01] = np.float32(1.4e-45)
        k = [100, 3000 if step == 0 else 7, 262]
        p.step(g, k, 0.0, tag=f"denorm p{path} s{step}")


def test_select_grid_option_rejects_bad_values():
    L = dgc.Learner([100], [10])
    for bad in (-1, 3):
        with pytest.raises(dgc.DGCError):
            L.set_option(dgc.DGC_OPT_SELECT_GRID, bad)
    for good in (0, 1, 2):
        L.set_option(dgc.DGC_OPT_SELECT_GRID, good)
    L.close()


@pytest.mark.parametrize("enc", ENCODE_PATHS)
@pytest.mark.parametrize("gap", [65534, 65535, 65536, 65537, 131072, 200000])
def test_encode_dense_tiles_with_one_long_gap(gap, enc):
    """Tiles of 1024 consecutive indices need no filler, and the count pass
    settles them from the tile's span alone; one gap of `gap` zeros lands
    inside the second tile (after entry 1500), another before the first
    entry of the fourth tile (entry 3072).  Streams against the oracle."""
    import torch
    n = 10000 + 2 * gap
    idx = np.concatenate([np.arange(1500), 1500 + gap + np.arange(1572),
                          3072 + 2 * gap + np.arange(1000)]).astype(np.uint32)
    assert idx[-1] < n and np.all(np.diff(idx.astype(np.int64)) > 0)
    val = np.random.default_rng(gap).standard_normal(idx.size).astype(np.float32)
    p = Pair([n], [idx.size])
    L = p.learner
    L.set_option(dgc.DGC_OPT_ENCODE_PATH, enc)
    L.idx[:idx.size].copy_(torch.from_numpy(idx.view(np.int32)))
    L.val[:idx.size].copy_(torch.from_numpy(val))
    got = gpu_streams(p, [idx.size])[0]
    want = oracle.encode(idx, val, cap=idx.size + n // 65536)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(f32_bits(got[1]), f32_bits(want[1]))
    assert L.status() == dgc.DGC_OK


def filler_heavy_indices(rng, k):
    """k sorted distinct indices: runs of neighbours and short gaps, with up
    to 12 gaps of one to three fillers' length at random entries (a filler
    offset that is not a multiple of 4 then carries into later tiles).
    Returns the indices and a tensor size that holds them."""
    gaps = rng.integers(0, 3, k).astype(np.int64)
    if k:
        at = rng.choice(k, min(k, 12), replace=False)
        gaps[at] = rng.integers(65535, 4 * 65536 + 2, at.size)
    pos = np.cumsum(gaps + 1) - 1
    n = int(pos[-1]) + 1 + int(rng.integers(0, 70000)) if k else int(rng.integers(1, 5000))
    return pos.astype(np.uint32), n


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_encode_paths_agree(seed):
    """Both encode paths (a workgroup per tensor, the tiled passes) and the
    automatic choice give the oracle's streams, through dgc_encode and
    through dgc_encode_counts, on layouts with empty, one-entry, ragged and
    many-tile tensors and with many fillers; the device-count variant with
    counts below the capacity."""
    import torch
    rng = np.random.default_rng(700 + seed)
    ks = [0, 1, 5, 1023, 1024, 1025, 4096, 4097, 9000, 3 * 1024 + 7]
    rng.shuffle(ks)
    made = [filler_heavy_indices(rng, k) for k in ks]
    idx = [m[0] for m in made]
    sizes = [m[1] for m in made]
    val = [rng.standard_normal(k).astype(np.float32) for k in ks]
    p = Pair(sizes, ks)
    L = p.learner
    L.idx[:sum(ks)].copy_(torch.from_numpy(np.concatenate(idx).view(np.int32)))
    L.val[:sum(ks)].copy_(torch.from_numpy(np.concatenate(val)))
    want = oracle_streams(sizes, ks, np.concatenate(idx), np.concatenate(val))
    assert sum(len(w[0]) for w in want) > sum(ks) + 50  # fillers present
    for enc in (0, 1, 2):
        say(f"encode paths seed {seed} enc {enc}")
        L.set_option(dgc.DGC_OPT_ENCODE_PATH, enc)
        L.runs.fill_(7)
        compare_streams(gpu_streams(p, ks), want, tag=f"seed{seed} enc{enc}")
        assert L.status() == dgc.DGC_OK
    # device counts: tensor t encodes its first c_t entries of the k_t slots
    cnt = [int(rng.integers(0, k + 1)) for k in ks]
    want_c = oracle_streams(sizes, cnt, np.concatenate([i[:c] for i, c in zip(idx, cnt)]),
                            np.concatenate([v[:c] for v, c in zip(val, cnt)]))
    for enc in (1, 2):
        say(f"encode counts seed {seed} enc {enc}")
        L.set_option(dgc.DGC_OPT_ENCODE_PATH, enc)
        L.count.copy_(torch.tensor(cnt, dtype=torch.int64))
        runs, vals, entries = L.encode_counts(ks)
        torch.cuda.synchronize()
        assert L.status() == dgc.DGC_OK
        r = runs.cpu().numpy().view(np.uint16)
        v = vals.cpu().numpy()
        e = entries.cpu().numpy()
        got = [(r[L.cap[t]:L.cap[t] + e[t]], v[L.cap[t]:L.cap[t] + e[t]])
               for t in range(len(sizes))]
        compare_streams(got, want_c, tag=f"seed{seed} counts enc{enc}")


def test_encode_path_option_rejects_bad_values():
    L = dgc.Learner([10], [1])
    for bad in (-1, 3):
        with pytest.raises(dgc.DGCError):
            L.set_option(dgc.DGC_OPT_ENCODE_PATH, bad)
    for good in (0, 1, 2):
        L.set_option(dgc.DGC_OPT_ENCODE_PATH, good)
    L.close()


@pytest.mark.parametrize("seed", [0, 1])
def test_codec_with_misaligned_buffers(seed):
    """Index, value, run and stream-value buffers one element past an aligned
    start (4-, 4-, 2- and 4-byte aligned, so no 8- or 16-byte access fits):
    both encode paths give the oracle's streams, and both scattered decode
    paths (spread passes, a workgroup per tensor) read them back into the
    oracle's sum."""
    import torch
    rng = np.random.default_rng(900 + seed)
    ks = [3, 1024, 1, 2051, 0, 700]
    made = [filler_heavy_indices(rng, k) for k in ks]
    idx = np.concatenate([m[0] for m in made])
    sizes = [m[1] for m in made]
    val = rng.standard_normal(idx.size).astype(np.float32)
    K = idx.size
    L = dgc.Learner(sizes, ks)
    C = int(L.cap[-1])
    ib = torch.zeros(K + 8, dtype=torch.int32, device="cuda")
    vb = torch.zeros(K + 8, dtype=torch.float32, device="cuda")
    ib[1:1 + K] = torch.from_numpy(idx.view(np.int32)).cuda()
    vb[1:1 + K] = torch.from_numpy(val).cuda()
    rb = torch.zeros(C + 16, dtype=torch.int16, device="cuda")
    sb = torch.zeros(C + 16, dtype=torch.float32, device="cuda")
    runs, svals = rb[1:1 + C], sb[1:1 + C]
    ent = torch.zeros(len(ks), dtype=torch.int64, device="cuda")
    assert ib[1:].data_ptr() % 16 and runs.data_ptr() % 8 and svals.data_ptr() % 16
    want = oracle_streams(sizes, ks, idx, val)
    n = sum(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)])
    dense0 = rng.standard_normal(n).astype(np.float32)
    want_sum = dense0.copy()
    for t, (wr, wv) in enumerate(want):
        assert oracle.decode_accumulate(wr, wv, want_sum[off[t]:off[t + 1]]) == 0
    for enc in (1, 2):
        say(f"misaligned codec seed {seed} enc {enc}")
        L.set_option(dgc.DGC_OPT_ENCODE_PATH, enc)
        rb.fill_(7)
        dgc.dgc_encode(L.state, ks, ib[1:], vb[1:], runs, svals, ent)
        torch.cuda.synchronize()
        assert L.status() == dgc.DGC_OK
        r = runs.cpu().numpy().view(np.uint16)
        s = svals.cpu().numpy()
        e = ent.cpu().numpy()
        got = [(r[L.cap[t]:L.cap[t] + e[t]], s[L.cap[t]:L.cap[t] + e[t]])
               for t in range(len(ks))]
        compare_streams(got, want, tag=f"misaligned enc{enc}")
        for path in (1, 3):
            L.set_option(dgc.DGC_OPT_DECODE_PATH, path)
            dense = torch.from_numpy(dense0.copy()).cuda()
            dgc.decode_accumulate(L, [(runs, svals, ent)], dense)
            torch.cuda.synchronize()
            assert L.status() == dgc.DGC_OK
            gd = dense.cpu().numpy()
            assert np.array_equal(f32_bits(gd), f32_bits(want_sum)), (
                enc, path, first_diff(gd, want_sum))
    L.close()
