"""dgc_shared_sum_static, the entry point that allocates nothing (for
callers that cannot allocate device memory): called through the raw C ABI,
its learner-order sums and fresh dense sum equal dgc_shared_sum's bit for
bit, on two calls in a row with the second one smaller, with more learners
than one pass adds, and with its status output for a corrupt index set."""

import ctypes

import numpy as np
import pytest

from gpu_harness import f32_bits, say
from sparsified_gradient_compression_amd import dgc
from sparsified_gradient_compression_amd import workloads as W

pytestmark = pytest.mark.gpu

MAX_TENSORS = 16384


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = dgc.lib()
    L.dgc_shared_sum_static.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
    L.dgc_shared_sum_static.restype = ctypes.c_int
    return torch


def static_call(sizes, vals, k, idx, out_sum, dense, status):
    import torch
    s = np.ascontiguousarray(sizes, np.int64)
    kk = np.ascontiguousarray(k, np.int64)
    Arr = ctypes.c_void_p * max(len(vals), 1)
    vv = Arr(*[x.data_ptr() for x in vals])
    return dgc.lib().dgc_shared_sum_static(
        len(s), s.ctypes.data, len(vals), ctypes.cast(vv, ctypes.c_void_p), kk.ctypes.data,
        idx.data_ptr() if idx is not None else None,
        out_sum.data_ptr() if out_sum is not None else None,
        dense.data_ptr() if dense is not None else None,
        status.data_ptr() if status is not None else None,
        torch.cuda.current_stream().cuda_stream)


def case(seed, sizes, density_den, n_learners):
    """Random shared index sets (ascending per tensor) and value vectors."""
    import torch
    rng = np.random.default_rng(seed)
    k = [-(-s // density_den) if s else 0 for s in sizes]
    idx = np.concatenate([np.sort(rng.choice(s, kk, replace=False)) if kk else
                          np.zeros(0, np.int64) for s, kk in zip(sizes, k)]).astype(np.uint32)
    K = int(sum(k))
    vals = []
    for _ in range(n_learners):
        x = rng.standard_normal(K).astype(np.float32)
        x[rng.random(K) < 0.05] = -0.0
        vals.append(torch.from_numpy(x).cuda())
    return k, torch.from_numpy(idx.view(np.int32)).cuda(), vals


def compare(sizes, k, idx, vals, tag):
    """dgc_shared_sum on a state of this layout against the static call."""
    import torch
    n, K = int(sum(sizes)), int(sum(k))
    L = dgc.Learner(list(sizes), k)
    ref_sum = torch.empty(max(K, 1), dtype=torch.float32, device="cuda")
    ref_dense = torch.full((max(n, 1),), float("nan"), dtype=torch.float32, device="cuda")
    dgc.shared_sum(L, vals, k, idx, ref_sum, ref_dense)
    out_sum = torch.full((max(K, 1) + 64,), 3.0, dtype=torch.float32, device="cuda")
    dense = torch.full((max(n, 1) + 64,), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    rc = static_call(sizes, vals, k, idx, out_sum, dense, status)
    assert rc == dgc.DGC_OK, (tag, rc)
    torch.cuda.synchronize()
    assert L.status() == dgc.DGC_OK
    assert int(status.cpu()[0]) == dgc.DGC_OK, tag
    assert np.array_equal(f32_bits(out_sum[:K].cpu().numpy()), f32_bits(ref_sum[:K].cpu().numpy())), tag
    assert np.array_equal(f32_bits(dense[:n].cpu().numpy()), f32_bits(ref_dense[:n].cpu().numpy())), tag
    assert (out_sum[K:].cpu().numpy() == 3.0).all() and np.isnan(dense[n:].cpu().numpy()).all()
    L.close()


def test_static_sum_equals_the_stateful_one_twice_second_smaller():
    big = list(W.scaled(W.get("resnet50"), 4).sizes)  # 161 tensors
    say("static sum: large call")
    k, idx, vals = case(61, big, 1000, 5)
    compare(big, k, idx, vals, "large")
    small = [70001, 3, 4096]
    say("static sum: smaller call")
    k, idx, vals = case(62, small, 50, 2)
    compare(small, k, idx, vals, "small")


def test_static_sum_many_learners_and_zero_learners():
    sizes = [300007, 1, 65536]
    k, idx, vals = case(63, sizes, 100, 40)
    compare(sizes, k, idx, vals, "40 learners")
    compare(sizes, k, idx, [], "no learners")


def test_static_sum_reports_a_corrupt_index_then_recovers():
    import torch
    sizes = [10000, 5000]
    k, idx, vals = case(64, sizes, 100, 3)
    bad = idx.clone()
    bad[-1] = 6000  # past the 5000-element tensor
    out_sum = torch.empty(sum(k), dtype=torch.float32, device="cuda")
    dense = torch.full((sum(sizes) + 64,), 5.0, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert static_call(sizes, vals, k, bad, out_sum, dense, status) == dgc.DGC_OK
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == dgc.DGC_ECORRUPT
    assert (dense[sum(sizes):].cpu().numpy() == 5.0).all()
    # the next call starts from a cleared latch
    compare(sizes, k, idx, vals, "after corrupt")


def test_static_sum_rejects_what_exceeds_its_scratch():
    import torch
    out_sum = torch.empty(1, dtype=torch.float32, device="cuda")
    sizes = [1] * (MAX_TENSORS + 1)
    k = [0] * (MAX_TENSORS + 1)
    assert static_call(sizes, [], k, None, out_sum, None, None) == dgc.DGC_ECAPACITY
    assert static_call([5], [], [6], None, out_sum, None, None) == dgc.DGC_EINVAL
    # exactly the maximum number of tensors is accepted
    sizes = [2] * MAX_TENSORS
    k = [1] * MAX_TENSORS
    kk, idx, vals = case(65, sizes, 2, 2)
    assert kk == k
    compare(sizes, k, idx, vals, "max tensors")
