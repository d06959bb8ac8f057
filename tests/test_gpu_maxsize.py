"""The largest tensor the C ABI accepts: n = 2**32 - 1 elements (local
indices are uint32), one tensor, in each of the three selectors.

The oracle cannot recompute a 16 GiB tensor within a test, so the checks are
properties that hold at any size and together fix the result: for exact
top-k, exactly k sent, every sent key >= every unsent key, ties at the
threshold taken in index order, sent + residual == accumulated v bitwise, u
= +0 exactly where sent; the stream decodes back to the sent entries.  For
the sampled threshold the sent set is {key >= theta, key != 0}; for the
bin-local rule it is the salient set computed with torch bin by bin.  The
gradient is drawn on the GPU with torch's seeded generator (Laplace, in
chunks), with exact ties and zeros planted.
"""

import numpy as np
import pytest

from gpu_harness import oracle_k, say
from sparsified_gradient_compression_amd import dgc

pytestmark = pytest.mark.gpu

N = (1 << 32) - 1
CHUNK = 1 << 28


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dgc.lib()
    import gc
    gc.collect()
    torch.cuda.empty_cache()  # memory cached by earlier test modules
    free, _ = torch.cuda.mem_get_info()
    if free < (200 << 30):
        pytest.skip("needs about 200 GiB of free device memory")
    return torch


def gradient(seed):
    """Laplace(0, 1e-3) in float32, plus planted ties (a run of equal
    magnitudes near the top) and exact zeros."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    g = torch.empty(N, dtype=torch.float32, device="cuda")
    for a in range(0, N, CHUNK):
        b = min(N, a + CHUNK)
        e = torch.empty(b - a, device="cuda").exponential_(1.0, generator=gen)
        sign = torch.rand(b - a, device="cuda", generator=gen) < 0.5
        g[a:b] = torch.where(sign, -e, e) * 1e-3
        del e, sign
    g[1000:3000] = 0.0
    g[N - 5000:N - 1000] = 9e-3   # equal magnitudes, near the top
    g[7:4000:3] = -9e-3
    return g


def keys_of(x):
    return x.view(__import__("torch").int32) & 0x7FFFFFFF


def local(idx, count):
    """uint32 local indices held in an int32 tensor, as int64."""
    return idx[:count].long() & 0xFFFFFFFF


def chunks():
    """Slices of at most 2**30 elements: some torch reductions and boolean
    indexing do not handle more than 2**31 elements at once."""
    step = 1 << 30
    for a in range(0, N, step):
        yield slice(a, min(N, a + step))


def bits(x):
    import torch
    return x.view(torch.int32)


def check_residual(L, sel, vals, u_new, v_new):
    """Sent values are v before masking; u = v = +0 where sent; everything
    else keeps the updated u and v bitwise.  Returns the sent mask."""
    import torch
    mask = torch.zeros(N, dtype=torch.bool, device="cuda")
    mask[sel] = True
    assert int(mask.sum()) == sel.numel()
    assert torch.equal(bits(vals), bits(v_new[sel]))
    for c in chunks():
        m = mask[c]
        for got, want in ((L.v[:N][c], v_new[c]), (L.u[:N][c], u_new[c])):
            assert bool(((bits(got) == 0) | ~m).all())
            assert bool(((bits(got) == bits(want)) | m).all())
    return mask


def check_roundtrip(L, sel, vals, encode):
    """The stream decodes (into zeros) to exactly the sent entries, and
    dgc_decode_sum gives the same bits over a buffer of NaNs."""
    import torch
    encode()
    dense = torch.zeros(N, dtype=torch.float32, device="cuda")
    dgc.decode_accumulate(L, [(L.runs, L.vals, L.entries)], dense)
    torch.cuda.synchronize()
    assert L.status() == dgc.DGC_OK
    want = torch.zeros(N, dtype=torch.float32, device="cuda")
    want[sel] = vals
    for c in chunks():
        assert torch.equal(bits(dense[c] + 0.0), bits(want[c] + 0.0))
    del want
    # the same stream as a fresh sum over NaNs: automatic path, then merged
    for path in (0, 2):
        L.set_option(dgc.DGC_OPT_DECODE_PATH, path)
        fresh = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        dgc.decode_sum(L, [(L.runs, L.vals, L.entries)], fresh)
        torch.cuda.synchronize()
        assert L.status() == dgc.DGC_OK
        for c in chunks():
            assert torch.equal(bits(fresh[c]), bits(dense[c])), path
        del fresh
    L.set_option(dgc.DGC_OPT_DECODE_PATH, 0)
    del dense


@pytest.mark.timeout(900)
def test_max_tensor_exact_topk():
    import torch
    k = oracle_k(N, __import__("fractions").Fraction(1, 1000))
    L = dgc.Learner([N], [k])
    for step in range(2):
        say(f"max size top-k step {step}: generate")
        g = gradient(100 + step)
        u_prev, v_prev = L.u[:N].clone(), L.v[:N].clone()
        say(f"max size top-k step {step}: compress")
        idx, val = L.compress(g, [k], 0.5)
        torch.cuda.synchronize()
        assert L.status() == dgc.DGC_OK
        # state update from the saved previous state
        s = L.scale.clone()
        m = torch.tensor(0.9, dtype=torch.float32, device="cuda")
        u_new = torch.add(torch.mul(m, u_prev), torch.mul(g, s))
        v_new = torch.add(v_prev, u_new)
        del u_prev, v_prev, g
        sel = local(idx, k)
        assert bool((sel[1:] > sel[:-1]).all()) and int(sel[-1]) < N
        mask = check_residual(L, sel, val[:k], u_new, v_new)
        kmin, kmax_un = 1 << 31, -1
        for c in chunks():
            key = keys_of(v_new[c])
            m = mask[c]
            kmin = min(kmin, int(torch.where(m, key, 0x7FFFFFFF).min()))
            kmax_un = max(kmax_un, int(torch.where(m, -1, key).max()))
        assert kmin >= kmax_un
        if kmin == kmax_un:  # ties at the threshold: the lower indices are sent
            last_sent, first_left = -1, N
            for c in chunks():
                tie = keys_of(v_new[c]) == kmin
                sent = torch.nonzero(tie & mask[c])
                left = torch.nonzero(tie & ~mask[c])
                if sent.numel():
                    last_sent = c.start + int(sent.max())
                if left.numel() and first_left == N:
                    first_left = c.start + int(left.min())
            assert last_sent < first_left
        del mask, u_new, v_new
        say(f"max size top-k step {step}: encode + decode")
        check_roundtrip(L, sel, val[:k].clone(), lambda: L.encode([k]))
        del sel
    L.close()


@pytest.mark.timeout(900)
def test_max_tensor_sampled_threshold():
    import torch
    k = N // 1000 + 1
    cap = 4 * k
    L = dgc.Learner([N], [cap])
    say("max size sampled: generate")
    g = gradient(200)
    u_prev, v_prev = L.u[:N].clone(), L.v[:N].clone()
    say("max size sampled: compress")
    idx, val, count, total = L.compress_sampled(g, [k], [cap], 0.5)
    torch.cuda.synchronize()
    assert L.status() == dgc.DGC_OK
    theta = int(L.select_info()[0, 4])
    c = int(count[0])
    assert c == int(total[0]) and 0.5 * k < c < 1.5 * k
    s = L.scale.clone()
    m = torch.tensor(0.9, dtype=torch.float32, device="cuda")
    u_new = torch.add(torch.mul(m, u_prev), torch.mul(g, s))
    v_new = torch.add(v_prev, u_new)
    del u_prev, v_prev, g
    sel = local(idx, c)
    mask = check_residual(L, sel, val[:c], u_new, v_new)
    for ch in chunks():
        key = keys_of(v_new[ch])
        assert torch.equal(mask[ch], (key >= theta) & (key != 0))
    del mask, u_new, v_new
    say("max size sampled: encode + decode")
    check_roundtrip(L, sel, val[:c].clone(), lambda: L.encode_counts([cap]))
    L.close()


@pytest.mark.timeout(900)
def test_max_tensor_binlocal():
    import torch
    Lb = 512
    cap = N // 8
    L = dgc.Learner([N], [cap])
    say("max size bin-local: generate")
    g = gradient(300)
    u_prev, v_prev = L.u[:N].clone(), L.v[:N].clone()
    say("max size bin-local: compress")
    idx, val, count, total = L.compress_binlocal(g, [Lb], [cap], 0.5)
    torch.cuda.synchronize()
    assert L.status() == dgc.DGC_OK
    c = int(count[0])
    assert c == int(total[0]) <= cap
    s = L.scale.clone()
    m = torch.tensor(0.9, dtype=torch.float32, device="cuda")
    u_new = torch.add(torch.mul(m, u_prev), torch.mul(g, s))
    v_new = torch.add(v_prev, u_new)
    del u_prev, v_prev, g
    sel = local(idx, c)
    mask = check_residual(L, sel, val[:c], u_new, v_new)
    # salient set bin by bin; chunks hold whole bins (2**30 is a multiple of
    # 512) and the last, short bin is padded with zero keys
    for ch in chunks():
        n = ch.stop - ch.start
        pad = (-n) % Lb
        key = torch.nn.functional.pad(keys_of(v_new[ch]), (0, pad)).view(-1, Lb)
        ahead = torch.nn.functional.pad(keys_of(torch.add(v_new[ch], u_new[ch])),
                                        (0, pad)).view(-1, Lb)
        theta = key.max(dim=1, keepdim=True).values
        salient = ((key != 0) & (ahead >= theta)).flatten()[:n]
        assert torch.equal(mask[ch], salient)
        del key, ahead, theta, salient
    del mask, u_new, v_new
    say("max size bin-local: encode + decode")
    check_roundtrip(L, sel, val[:c].clone(), lambda: L.encode_counts([cap]))
    L.close()
