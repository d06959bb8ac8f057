"""GPU parity of dgc_decode_accumulate on its paths: each learner's stream
added on its own (by passes spread over 1024-entry tiles, or by one
workgroup per tensor for a batch of learners), and the merged pass (dense
blocks held on chip, learners added in order) -- forced each way and
automatic.  Streams are
encoded by the oracle from seeded random selections at densities from 30%
down to 0.1%; the dense sum starts from random values (and -0.0), so the
order of the additions is visible in the bits.  The reference is the
oracle's decoder run learner after learner.
"""

import numpy as np
import pytest

import oracle
from gpu_harness import f32_bits, first_diff, say
from sparsified_gradient_compression_amd import dgc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dgc.lib()
    return torch


def make_streams(rng, sizes, densities, cap):
    """Per learner: oracle-encoded (runs, vals) per tensor, and the device
    buffers laid out at the capacity offsets."""
    import torch
    C = int(cap[-1])
    out = []
    for d in densities:
        runs = np.zeros(max(C, 1), np.uint16)
        vals = np.zeros(max(C, 1), np.float32)
        ent = np.zeros(len(sizes), np.int64)
        per = []
        for t, n in enumerate(sizes):
            k = int(rng.binomial(n, d)) if n else 0
            k = min(k, int(cap[t + 1] - cap[t]) - n // 65536)
            idx = np.sort(rng.choice(n, size=k, replace=False)).astype(np.uint32) if k else \
                np.zeros(0, np.uint32)
            val = rng.standard_normal(k).astype(np.float32)
            val[rng.random(k) < 0.05] = -0.0
            r, v = oracle.encode(idx, val, cap=int(cap[t + 1] - cap[t]))
            runs[cap[t]:cap[t] + r.size] = r
            vals[cap[t]:cap[t] + r.size] = v
            ent[t] = r.size
            per.append((r, v))
        out.append((per, torch.from_numpy(runs.view(np.int16)).cuda(),
                    torch.from_numpy(vals).cuda(), torch.from_numpy(ent).cuda()))
    return out


def reference(sizes, dense0, streams):
    want = dense0.copy()
    off = np.concatenate([[0], np.cumsum(sizes)])
    for per, *_ in streams:
        for t, (r, v) in enumerate(per):
            assert oracle.decode_accumulate(r, v, want[off[t]:off[t + 1]]) == 0
    return want


def decode(L, streams, dense0, path):
    import torch
    L.set_option(dgc.DGC_OPT_DECODE_PATH, path)
    dense = torch.from_numpy(dense0.copy()).cuda()
    dgc.decode_accumulate(L, [(s[1], s[2], s[3]) for s in streams], dense)
    torch.cuda.synchronize()
    return dense.cpu().numpy()


LAYOUTS = [
    [1, 4095, 4096, 4097, 8192 + 3, 70001],
    [1 << 20],
    [0, 7, 65536, 65537, 131073, 300007, 5],
]


@pytest.mark.parametrize("layout", range(len(LAYOUTS)))
@pytest.mark.parametrize("W,dens", [(1, [0.3]), (2, [0.05, 0.2]), (4, [0.05] * 4),
                                    (5, [0.001, 0.3, 0.01, 0.1, 0.05]),
                                    (9, [0.02] * 9), (17, [0.07] * 17)])
def test_decode_paths_match_oracle(layout, W, dens):
    sizes = LAYOUTS[layout]
    rng = np.random.default_rng([91, layout, W])
    L = dgc.Learner(sizes, sizes)
    streams = make_streams(rng, sizes, dens, L.cap)
    n = sum(sizes)
    dense0 = rng.standard_normal(max(n, 1)).astype(np.float32)
    dense0[rng.random(dense0.size) < 0.1] = -0.0
    want = reference(sizes, dense0[:n], streams)
    for path in (1, 2, 3, 0):
        say(f"decode layout {layout} W={W} path {path}")
        got = decode(L, streams, dense0, path)[:n]
        assert L.status() == dgc.DGC_OK
        assert np.array_equal(f32_bits(got), f32_bits(want)), (path, first_diff(got, want))


def test_merged_decode_flags_corrupt_streams():
    """A stream that walks past its tensor's end, or claims more entries
    than its capacity, is flagged on the merged path too, and nothing is
    written outside the tensor."""
    import torch
    sizes = [10000, 5000]
    L = dgc.Learner(sizes, sizes)
    rng = np.random.default_rng(92)
    streams = make_streams(rng, sizes, [0.3, 0.3], L.cap)
    # learner 1, tensor 0: runs that pass the end of the 10000-element tensor
    per, runs, vals, ent = streams[1]
    r = runs.cpu().numpy().view(np.uint16).copy()
    r[L.cap[0]:L.cap[0] + int(ent[0])] = 200
    streams[1] = (per, torch.from_numpy(r.view(np.int16)).cuda(), vals, ent)
    guard = 123.0
    dense0 = np.full(sum(sizes) + 64, guard, np.float32)
    got = decode(L, streams, dense0, 2)
    assert L.status() == dgc.DGC_ECORRUPT
    assert (got[sum(sizes):] == guard).all()
    # entry count above capacity
    per, runs, vals, ent = streams[0]
    bad = ent.clone()
    bad[1] = int(L.cap[2] - L.cap[1]) + 1
    streams[0] = (per, runs, vals, bad)
    decode(L, streams, dense0, 2)
    assert L.status() == dgc.DGC_ECORRUPT
    assert L.status() == dgc.DGC_OK


def test_decode_option_rejects_bad_values():
    L = dgc.Learner([100], [10])
    with pytest.raises(dgc.DGCError):
        L.set_option(dgc.DGC_OPT_DECODE_PATH, 4)
    with pytest.raises(dgc.DGCError):
        L.set_option(dgc.DGC_OPT_DECODE_PATH, -1)
    for good in (0, 1, 2, 3):
        L.set_option(dgc.DGC_OPT_DECODE_PATH, good)


def decode_fresh(L, streams, n, path, guard=None):
    """dgc_decode_sum into a buffer that holds NaNs, -0.0 and random values
    (and, past n, a guard value that must survive)."""
    import torch
    L.set_option(dgc.DGC_OPT_DECODE_PATH, path)
    rng = np.random.default_rng(n + 5)
    junk = rng.standard_normal(n + 64).astype(np.float32)
    junk[::7] = np.nan
    junk[::11] = -0.0
    if guard is not None:
        junk[n:] = guard
    dense = torch.from_numpy(junk).cuda()
    dgc.decode_sum(L, [(s[1], s[2], s[3]) for s in streams], dense)
    torch.cuda.synchronize()
    return dense.cpu().numpy()


@pytest.mark.parametrize("layout", range(len(LAYOUTS)))
@pytest.mark.parametrize("W,dens", [(0, []), (1, [0.3]), (1, [0.001]),
                                    (4, [0.001] * 4), (5, [0.001, 0.3, 0.01, 0.1, 0.05]),
                                    (9, [0.02] * 9), (17, [0.07] * 17)])
def test_decode_sum_matches_oracle(layout, W, dens):
    """dgc_decode_sum = the oracle's decode of every learner onto +0.0, bit for
    bit, whatever dense held; the decode-path option only steers learners
    past the first 8."""
    sizes = LAYOUTS[layout]
    rng = np.random.default_rng([93, layout, W])
    L = dgc.Learner(sizes, sizes)
    streams = make_streams(rng, sizes, dens, L.cap)
    n = sum(sizes)
    want = reference(sizes, np.zeros(n, np.float32), streams)
    for path in (1, 2, 3, 0):
        say(f"decode_sum layout {layout} W={W} path {path}")
        got = decode_fresh(L, streams, n, path, guard=77.0)
        assert L.status() == dgc.DGC_OK
        assert np.array_equal(f32_bits(got[:n]), f32_bits(want)), (path, first_diff(got[:n], want))
        assert (got[n:] == 77.0).all()


def test_decode_sum_without_capacity():
    """A layout whose streams have no capacity at all (k = 0, tensors under
    65536 elements): the fresh sum is all +0.0."""
    sizes = [100, 3, 65535]
    L = dgc.Learner(sizes, [0, 0, 0])
    assert int(L.cap[-1]) == 0
    streams = make_streams(np.random.default_rng(94), sizes, [0.1, 0.1], L.cap)
    n = sum(sizes)
    got = decode_fresh(L, streams, n, 0, guard=5.0)
    assert L.status() == dgc.DGC_OK
    assert (f32_bits(got[:n]) == 0).all()
    assert (got[n:] == 5.0).all()


@pytest.mark.parametrize("path", [0, 3])
def test_decode_sum_flags_corrupt_streams(path):
    import torch
    sizes = [10000, 5000]
    L = dgc.Learner(sizes, sizes)
    rng = np.random.default_rng(95)
    streams = make_streams(rng, sizes, [0.3, 0.3], L.cap)
    per, runs, vals, ent = streams[1]
    r = runs.cpu().numpy().view(np.uint16).copy()
    r[L.cap[0]:L.cap[0] + int(ent[0])] = 200
    streams[1] = (per, torch.from_numpy(r.view(np.int16)).cuda(), vals, ent)
    got = decode_fresh(L, streams, sum(sizes), path, guard=123.0)
    assert L.status() == dgc.DGC_ECORRUPT
    assert (got[sum(sizes):] == 123.0).all()
    assert np.isfinite(got[:sum(sizes)]).all()  # every element written
    assert L.status() == dgc.DGC_OK


@pytest.mark.parametrize("path", [0, 1, 2, 3])
@pytest.mark.parametrize("shift", [1, 2, 3])
def test_decode_sum_into_unaligned_dense(path, shift):
    """The dense sum may start at any 4-byte boundary: a view `shift`
    elements into a buffer of NaNs, with guards on both sides.  The
    zero-fill's head and tail and the merge's element-wise stores (no
    16-byte block) are exercised; the result is the oracle's."""
    import torch
    sizes = [4096 * 5 + 3, 65536 + 1024, 7]
    rng = np.random.default_rng([96, path, shift])
    L = dgc.Learner(sizes, sizes)
    L.set_option(dgc.DGC_OPT_DECODE_PATH, path)
    streams = make_streams(rng, sizes, [0.05, 0.2, 0.001], L.cap)
    n = sum(sizes)
    want = reference(sizes, np.zeros(n, np.float32), streams)
    buf = torch.full((n + 64,), float("nan"), dtype=torch.float32, device="cuda")
    buf[:shift] = 11.0
    buf[shift + n:] = 22.0
    dense = buf[shift:shift + n]
    assert dense.data_ptr() % 16 != 0
    dgc.decode_sum(L, [(s[1], s[2], s[3]) for s in streams], dense)
    torch.cuda.synchronize()
    assert L.status() == dgc.DGC_OK
    got = buf.cpu().numpy()
    assert np.array_equal(f32_bits(got[shift:shift + n]), f32_bits(want)), first_diff(
        got[shift:shift + n], want)
    assert (got[:shift] == 11.0).all() and (got[shift + n:] == 22.0).all()


@pytest.mark.parametrize("W", [2, 4, 9])
def test_decode_sum_small_capacity_mixed_layout(W):
    """A fresh sum whose layout is mostly sparse (a 2^20 tensor with room for
    n/10000 entries) but holds one small dense tensor (64 elements, full
    capacity): the library zero-fills dense first and then merges only the
    tensors whose streams are dense enough.  Bit for bit the oracle's
    decode onto +0.0 on every path setting."""
    sizes = [64, 1 << 20, 3]
    kmax = [64, (1 << 20) // 10000, 3]
    rng = np.random.default_rng([97, W])
    L = dgc.Learner(sizes, kmax)
    streams = make_streams(rng, sizes, [0.3] * W, L.cap)
    n = sum(sizes)
    want = reference(sizes, np.zeros(n, np.float32), streams)
    for path in (0, 1, 2, 3):
        say(f"decode_sum small capacity W={W} path {path}")
        got = decode_fresh(L, streams, n, path, guard=9.0)
        assert L.status() == dgc.DGC_OK
        assert np.array_equal(f32_bits(got[:n]), f32_bits(want)), (path, first_diff(got[:n], want))
        assert (got[n:] == 9.0).all()


@pytest.mark.parametrize("path", [1, 3])
def test_scattered_decode_of_corrupt_streams_matches_oracle(path):
    """On both scattered paths a stream that walks past its tensor's end adds
    its entries up to that point (as the oracle's decoder does) and is
    flagged; one whose entry count exceeds its capacity adds nothing for
    that tensor and is flagged; the other streams add as usual, in learner
    order."""
    import torch
    sizes = [3000, 70001, 5]
    L = dgc.Learner(sizes, [300, 200, 5])
    rng = np.random.default_rng([98, path])
    streams = make_streams(rng, sizes, [0.05] * 3, L.cap)  # per learner
    off = np.concatenate([[0], np.cumsum(sizes)])
    # learner 1, tensor 0: every run 40, so the walk passes 3000 part-way
    per, runs, vals, ent = streams[1]
    r = runs.cpu().numpy().view(np.uint16).copy()
    e0 = int(ent[0])
    assert 41 * e0 > sizes[0]
    r[L.cap[0]:L.cap[0] + e0] = 40
    streams[1] = (per, torch.from_numpy(r.view(np.int16)).cuda(), vals, ent)
    # learner 2, tensor 1: an entry count above the capacity
    per2, runs2, vals2, ent2 = streams[2]
    bad = ent2.clone()
    bad[1] = int(L.cap[2] - L.cap[1]) + 1
    streams[2] = (per2, runs2, vals2, bad)
    dense0 = rng.standard_normal(sum(sizes)).astype(np.float32)
    want = dense0.copy()
    for w, (_, rr, vv, ee) in enumerate(streams):
        rh = rr.cpu().numpy().view(np.uint16)
        vh = vv.cpu().numpy()
        eh = ee.cpu().numpy()
        for t in range(len(sizes)):
            cap_t = int(L.cap[t + 1] - L.cap[t])
            if eh[t] < 0 or eh[t] > cap_t:
                continue
            a = int(L.cap[t])
            rc = oracle.decode_accumulate(rh[a:a + eh[t]].copy(), vh[a:a + eh[t]].copy(),
                                          want[off[t]:off[t + 1]])
            assert rc == (-1 if (w, t) == (1, 0) else 0)
    got = decode(L, streams, dense0, path)
    assert L.status() == dgc.DGC_ECORRUPT
    assert L.status() == dgc.DGC_OK
    assert np.array_equal(f32_bits(got), f32_bits(want)), first_diff(got, want)


@pytest.mark.parametrize("W", [1, 2, 4, 8, 9])
def test_decode_small_capacity_layouts_every_path(W):
    """Layouts whose streams hold few tiles per tensor (the automatic choice
    takes one workgroup per tensor for up to 8 tiles per tensor and batch):
    accumulate and fresh sums on every path setting, bit for bit the
    oracle's decode in learner order."""
    sizes = [1 << 20, 5000, 70001, 1, 0, 2359296]
    kmax = [1049, 5, 71, 1, 0, 2360]
    rng = np.random.default_rng([99, W])
    L = dgc.Learner(sizes, kmax)
    streams = make_streams(rng, sizes, [0.001] * W, L.cap)
    n = sum(sizes)
    dense0 = rng.standard_normal(n).astype(np.float32)
    dense0[rng.random(n) < 0.1] = -0.0
    want_acc = reference(sizes, dense0, streams)
    want_fresh = reference(sizes, np.zeros(n, np.float32), streams)
    for path in (0, 1, 2, 3):
        say(f"decode small capacity W={W} path {path}")
        got = decode(L, streams, dense0, path)
        assert L.status() == dgc.DGC_OK
        assert np.array_equal(f32_bits(got), f32_bits(want_acc)), (path, first_diff(got, want_acc))
        got = decode_fresh(L, streams, n, path, guard=3.0)
        assert L.status() == dgc.DGC_OK
        assert np.array_equal(f32_bits(got[:n]), f32_bits(want_fresh)), (
            path, first_diff(got[:n], want_fresh))
        assert (got[n:] == 3.0).all()
