"""GPU parity at the full workload sizes.

resnet50 (25.6M, 161 tensors, 10 steps), deepspeech (122M, 4 learners) and
warmup350m (350M, k from 87.5M down to 350k) are compared with the oracle in
full.  flat1b (2**30 elements in 64 chunks, 4 learners x 3 steps) runs in
the launch configuration the benchmark times; the oracle recomputes four
sampled chunks per learner-step in full (its norm is over the whole
gradient), and properties that hold at any size are checked on every chunk.
"""

import numpy as np
import pytest

import oracle
from gpu_harness import f32_bits, first_diff, say
from sparsified_gradient_compression_amd import dgc
from sparsified_gradient_compression_amd import workloads as W
from test_gpu_parity import run_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dgc.lib()
    return torch


@pytest.mark.timeout(600)
def test_resnet50_full():
    run_workload(W.get("resnet50"), tag="rn50")


@pytest.mark.timeout(600)
def test_deepspeech_full():
    run_workload(W.get("deepspeech"), tag="ds")


@pytest.mark.timeout(900)
def test_warmup350m_full():
    run_workload(W.get("warmup350m"), tag="warm350m")


SAMPLED = (0, 17, 42, 63)


@pytest.mark.timeout(1200)
def test_flat1b_full_sampled():
    import torch
    wl = W.get("flat1b")
    C = wl.sizes[0]
    T = len(wl.sizes)
    k = [dgc.k_for_density(C, wl.densities[0])] * T
    assert k[0] == 16778
    m = np.float32(wl.momentum)
    learners = [dgc.Learner(list(wl.sizes), k, wl.momentum) for _ in range(wl.learners)]
    # oracle state of the sampled chunks, per learner
    ou = [{c: np.zeros(C, np.float32) for c in SAMPLED} for _ in learners]
    ov = [{c: np.zeros(C, np.float32) for c in SAMPLED} for _ in learners]
    g_host = np.empty(wl.n, np.float32)
    for t in range(wl.steps):
        o_streams = []  # per learner: {chunk: (runs, vals)}
        for w, L in enumerate(learners):
            say(f"flat1b step {t} learner {w}: generate")
            W.gradient(wl, w, t, out=g_host)
            g = torch.from_numpy(g_host).cuda()
            u_prev = L.u.clone()
            v_prev = L.v.clone()
            say(f"flat1b step {t} learner {w}: compress")
            idx, val = L.compress(g, k, wl.clip)
            L.encode(k)
            torch.cuda.synchronize()
            assert L.status() == dgc.DGC_OK
            assert L.path_counts() == (T, 0)
            norm = float(L.norm.cpu()[0])
            s = np.float32(L.scale.cpu()[0])
            # ---- oracle on the sampled chunks
            o_norm, o_s = oracle.clip_scale(g_host, wl.clip)
            assert abs(norm - o_norm) <= 1e-6 * o_norm and s == o_s, (norm, o_norm, s, o_s)
            gi = idx.cpu().numpy().view(np.uint32).reshape(T, k[0])
            gvv = val.cpu().numpy().reshape(T, k[0])
            cap = L.cap
            runs = L.runs.cpu().numpy().view(np.uint16)
            svals = L.vals.cpu().numpy()
            ent = L.entries.cpu().numpy()
            o_streams.append({})
            for c in SAMPLED:
                sl = slice(c * C, (c + 1) * C)
                oracle.momentum(g_host[sl], o_s, m, ou[w][c], ov[w][c])
                o_idx, o_val = oracle.select_mask(ou[w][c], ov[w][c], k[0])
                assert np.array_equal(gi[c], o_idx), (t, w, c, first_diff(gi[c], o_idx))
                assert np.array_equal(f32_bits(gvv[c]), f32_bits(o_val)), (t, w, c)
                assert np.array_equal(f32_bits(L.u[sl].cpu().numpy()), f32_bits(ou[w][c]))
                assert np.array_equal(f32_bits(L.v[sl].cpu().numpy()), f32_bits(ov[w][c]))
                o_r, o_v = oracle.encode(o_idx, o_val, cap=int(cap[c + 1] - cap[c]))
                assert ent[c] == o_r.size
                assert np.array_equal(runs[cap[c]:cap[c] + ent[c]], o_r)
                assert np.array_equal(f32_bits(svals[cap[c]:cap[c] + ent[c]]), f32_bits(o_v))
                o_streams[-1][c] = (o_r, o_v)
            # ---- properties on every chunk (torch on the GPU, separate ops:
            # no contraction)
            sd = torch.tensor(float(s), dtype=torch.float32, device="cuda")
            md = torch.tensor(float(m), dtype=torch.float32, device="cuda")
            u_new = torch.add(torch.mul(md, u_prev), torch.mul(g, sd))
            v_pre = torch.add(v_prev, u_new)
            del u_prev, v_prev
            gidx = idx.long().view(T, k[0]) + torch.arange(T, device="cuda").view(T, 1) * C
            assert bool((gidx[:, 1:] > gidx[:, :-1]).all())
            gidx = gidx.flatten()
            sent = torch.zeros_like(v_pre)
            sent[gidx] = val
            # sent + residual == accumulated v, bitwise
            assert torch.equal((sent + L.v[: wl.n]).view(torch.int32),
                               (v_pre + 0.0).view(torch.int32))
            mask = torch.zeros(wl.n, dtype=torch.bool, device="cuda")
            mask[gidx] = True
            assert bool((L.u[: wl.n][mask] == 0).all())
            assert torch.equal(L.u[: wl.n][~mask].view(torch.int32),
                               u_new[~mask].view(torch.int32))
            keys = (v_pre.view(torch.int32) & 0x7FFFFFFF).view(T, C)
            top = torch.topk(keys, k[0], dim=1).values
            got_keys = (val.view(torch.int32) & 0x7FFFFFFF).view(T, k[0])
            assert torch.equal(torch.sort(top, dim=1).values,
                               torch.sort(got_keys, dim=1).values)
            del sent, mask, keys, top, v_pre, u_new, g
        # ---- decode of the four learners' streams, in learner order
        say(f"flat1b step {t}: decode")
        dense = torch.zeros(wl.n, dtype=torch.float32, device="cuda")
        dgc.decode_accumulate(learners[0], [(L.runs, L.vals, L.entries) for L in learners],
                              dense)
        torch.cuda.synchronize()
        assert learners[0].status() == dgc.DGC_OK
        for c in SAMPLED:
            want = np.zeros(C, np.float32)
            for w in range(len(learners)):
                r, v_ = o_streams[w][c]
                assert oracle.decode_accumulate(r, v_, want) == 0
            got = dense[c * C:(c + 1) * C].cpu().numpy()
            assert np.array_equal(f32_bits(got), f32_bits(want)), (t, c)
        ref = torch.zeros_like(dense)
        for L in learners:
            gi = L.idx.long().view(T, k[0]) + torch.arange(T, device="cuda").view(T, 1) * C
            gi = gi.flatten()
            ref[gi] = ref[gi] + L.val
        assert torch.equal(ref, dense)

        # the fresh sum the benchmark times: dgc_decode_sum into a buffer of NaNs
        fresh = torch.full_like(dense, float("nan"))
        dgc.decode_sum(learners[0], [(L.runs, L.vals, L.entries) for L in learners], fresh)
        torch.cuda.synchronize()
        assert learners[0].status() == dgc.DGC_OK
        assert torch.equal(fresh.view(torch.int32), dense.view(torch.int32)), t
        del fresh
        del dense, ref


@pytest.mark.timeout(1200)
def test_flat1b_binlocal_full_sampled():
    """The bin-local selector (AdaComp page) at full size in the benchmark's
    configuration: bins of 512, at most n_t/8 entries per chunk, 4 learners
    x 3 steps.  The oracle recomputes four sampled chunks per learner-step;
    on every chunk: delivered = min(salient, cap), the delivered set is the
    salient set (none truncated here) found independently with torch, sent +
    residual == accumulated v bitwise, u = +0 exactly where sent."""
    import torch
    wl = W.get("flat1b")
    C = wl.sizes[0]
    T = len(wl.sizes)
    Lb = 512
    cap = [C // 8] * T
    m = np.float32(wl.momentum)
    learners = [dgc.Learner(list(wl.sizes), cap, wl.momentum) for _ in range(wl.learners)]
    ou = [{c: np.zeros(C, np.float32) for c in SAMPLED} for _ in learners]
    ov = [{c: np.zeros(C, np.float32) for c in SAMPLED} for _ in learners]
    g_host = np.empty(wl.n, np.float32)
    coff = np.arange(T + 1) * cap[0]
    for t in range(wl.steps):
        o_streams = []
        for w, L in enumerate(learners):
            say(f"flat1b binlocal step {t} learner {w}: generate")
            W.gradient(wl, w, t, out=g_host)
            g = torch.from_numpy(g_host).cuda()
            u_prev = L.u.clone()
            v_prev = L.v.clone()
            say(f"flat1b binlocal step {t} learner {w}: compress")
            idx, val, count, total = L.compress_binlocal(g, [Lb] * T, cap, wl.clip)
            L.encode_counts(cap)
            torch.cuda.synchronize()
            assert L.status() == dgc.DGC_OK
            cnt = count.cpu().numpy()
            tot = total.cpu().numpy()
            assert np.array_equal(cnt, np.minimum(tot, cap[0])) and (tot <= cap[0]).all()
            s = np.float32(L.scale.cpu()[0])
            o_norm, o_s = oracle.clip_scale(g_host, wl.clip)
            assert s == o_s
            gi = idx.cpu().numpy().view(np.uint32)
            gvv = val.cpu().numpy()
            scap = L.cap
            runs = L.runs.cpu().numpy().view(np.uint16)
            svals = L.vals.cpu().numpy()
            ent = L.entries.cpu().numpy()
            o_streams.append({})
            for c in SAMPLED:
                sl = slice(c * C, (c + 1) * C)
                oracle.momentum(g_host[sl], o_s, m, ou[w][c], ov[w][c])
                o_idx, o_val, o_tot = oracle.binlocal_select_mask(ou[w][c], ov[w][c], Lb,
                                                                  cap[c])
                a = coff[c]
                assert tot[c] == o_tot and cnt[c] == o_idx.size, (t, w, c)
                assert np.array_equal(gi[a:a + cnt[c]], o_idx), (t, w, c)
                assert np.array_equal(f32_bits(gvv[a:a + cnt[c]]), f32_bits(o_val)), (t, w, c)
                assert np.array_equal(f32_bits(L.u[sl].cpu().numpy()), f32_bits(ou[w][c]))
                assert np.array_equal(f32_bits(L.v[sl].cpu().numpy()), f32_bits(ov[w][c]))
                o_r, o_v = oracle.encode(o_idx, o_val, cap=int(scap[c + 1] - scap[c]))
                assert ent[c] == o_r.size
                assert np.array_equal(runs[scap[c]:scap[c] + ent[c]], o_r)
                assert np.array_equal(f32_bits(svals[scap[c]:scap[c] + ent[c]]), f32_bits(o_v))
                o_streams[-1][c] = (o_r, o_v)
            # ---- properties on every chunk (torch, separate ops: no contraction)
            sd = torch.tensor(float(s), dtype=torch.float32, device="cuda")
            md = torch.tensor(float(m), dtype=torch.float32, device="cuda")
            u_new = torch.add(torch.mul(md, u_prev), torch.mul(g, sd))
            v_pre = torch.add(v_prev, u_new)
            del u_prev, v_prev, g
            key = (v_pre.view(torch.int32) & 0x7FFFFFFF).view(-1, Lb)
            ahead = (torch.add(v_pre, u_new).view(torch.int32) & 0x7FFFFFFF).view(-1, Lb)
            theta = key.max(dim=1, keepdim=True).values
            salient = ((key != 0) & (ahead >= theta)).flatten()
            del key, ahead, theta
            assert int(salient.sum()) == int(tot.sum())
            sel = torch.cat([idx[coff[c]:coff[c] + cnt[c]].long() + c * C for c in range(T)])
            vsel = torch.cat([val[coff[c]:coff[c] + cnt[c]] for c in range(T)])
            mask = torch.zeros(wl.n, dtype=torch.bool, device="cuda")
            mask[sel] = True
            assert torch.equal(mask, salient)
            sent = torch.zeros_like(v_pre)
            sent[sel] = vsel
            assert torch.equal((sent + L.v[: wl.n]).view(torch.int32),
                               (v_pre + 0.0).view(torch.int32))
            assert bool((L.u[: wl.n][mask].view(torch.int32) == 0).all())
            assert torch.equal(L.u[: wl.n][~mask].view(torch.int32),
                               u_new[~mask].view(torch.int32))
            del sent, mask, salient, sel, vsel, v_pre, u_new
        say(f"flat1b binlocal step {t}: decode")
        dense = torch.zeros(wl.n, dtype=torch.float32, device="cuda")
        dgc.decode_accumulate(learners[0], [(L.runs, L.vals, L.entries) for L in learners],
                              dense)
        torch.cuda.synchronize()
        assert learners[0].status() == dgc.DGC_OK
        for c in SAMPLED:
            want = np.zeros(C, np.float32)
            for w in range(len(learners)):
                r, v_ = o_streams[w][c]
                assert oracle.decode_accumulate(r, v_, want) == 0
            got = dense[c * C:(c + 1) * C].cpu().numpy()
            assert np.array_equal(f32_bits(got), f32_bits(want)), (t, c)

        # the fresh sum the benchmark times: dgc_decode_sum into a buffer of NaNs
        fresh = torch.full_like(dense, float("nan"))
        dgc.decode_sum(learners[0], [(L.runs, L.vals, L.entries) for L in learners], fresh)
        torch.cuda.synchronize()
        assert learners[0].status() == dgc.DGC_OK
        assert torch.equal(fresh.view(torch.int32), dense.view(torch.int32)), t
        del fresh
        del dense


@pytest.mark.timeout(1200)
def test_flat1b_sampled_full_sampled():
    """The sampled-threshold selector (DGC review, RQ4) at full size in the
    benchmark's configuration: k = 16778 per chunk, at most 4 k delivered,
    4 learners x 3 steps.  The oracle recomputes four sampled chunks per
    learner-step (threshold, sent set, state, stream); on every chunk the
    sent set is {key >= theta, key != 0} found with torch, the residual and
    masking hold bitwise, and the count stays within 0.5 k .. 1.5 k."""
    import torch
    wl = W.get("flat1b")
    C = wl.sizes[0]
    T = len(wl.sizes)
    k = [dgc.k_for_density(C, wl.densities[0])] * T
    cap = [4 * k[0]] * T
    m = np.float32(wl.momentum)
    learners = [dgc.Learner(list(wl.sizes), cap, wl.momentum) for _ in range(wl.learners)]
    ou = [{c: np.zeros(C, np.float32) for c in SAMPLED} for _ in learners]
    ov = [{c: np.zeros(C, np.float32) for c in SAMPLED} for _ in learners]
    g_host = np.empty(wl.n, np.float32)
    coff = np.arange(T + 1) * cap[0]
    for t in range(wl.steps):
        o_streams = []
        for w, L in enumerate(learners):
            say(f"flat1b sampled step {t} learner {w}: generate")
            W.gradient(wl, w, t, out=g_host)
            g = torch.from_numpy(g_host).cuda()
            u_prev = L.u.clone()
            v_prev = L.v.clone()
            say(f"flat1b sampled step {t} learner {w}: compress")
            idx, val, count, total = L.compress_sampled(g, k, cap, wl.clip)
            L.encode_counts(cap)
            torch.cuda.synchronize()
            assert L.status() == dgc.DGC_OK
            info = L.select_info()
            assert (info[:, 0] == 3).all()
            theta = info[:, 4]
            cnt = count.cpu().numpy()
            tot = total.cpu().numpy()
            assert np.array_equal(cnt, np.minimum(tot, cap[0]))
            assert (tot > k[0] // 2).all() and (tot < 3 * k[0] // 2).all(), (tot.min(), tot.max())
            s = np.float32(L.scale.cpu()[0])
            _, o_s = oracle.clip_scale(g_host, wl.clip)
            assert s == o_s
            gi = idx.cpu().numpy().view(np.uint32)
            gvv = val.cpu().numpy()
            scap = L.cap
            runs = L.runs.cpu().numpy().view(np.uint16)
            svals = L.vals.cpu().numpy()
            ent = L.entries.cpu().numpy()
            o_streams.append({})
            for c in SAMPLED:
                sl = slice(c * C, (c + 1) * C)
                oracle.momentum(g_host[sl], o_s, m, ou[w][c], ov[w][c])
                o_idx, o_val, o_tot, o_th = oracle.sampled_select_mask(ou[w][c], ov[w][c],
                                                                       k[c], c, cap[c])
                a = coff[c]
                assert theta[c] == o_th and tot[c] == o_tot, (t, w, c)
                assert np.array_equal(gi[a:a + cnt[c]], o_idx), (t, w, c)
                assert np.array_equal(f32_bits(gvv[a:a + cnt[c]]), f32_bits(o_val)), (t, w, c)
                assert np.array_equal(f32_bits(L.u[sl].cpu().numpy()), f32_bits(ou[w][c]))
                assert np.array_equal(f32_bits(L.v[sl].cpu().numpy()), f32_bits(ov[w][c]))
                o_r, o_v = oracle.encode(o_idx, o_val, cap=int(scap[c + 1] - scap[c]))
                assert ent[c] == o_r.size
                assert np.array_equal(runs[scap[c]:scap[c] + ent[c]], o_r)
                assert np.array_equal(f32_bits(svals[scap[c]:scap[c] + ent[c]]), f32_bits(o_v))
                o_streams[-1][c] = (o_r, o_v)
            sd = torch.tensor(float(s), dtype=torch.float32, device="cuda")
            md = torch.tensor(float(m), dtype=torch.float32, device="cuda")
            u_new = torch.add(torch.mul(md, u_prev), torch.mul(g, sd))
            v_pre = torch.add(v_prev, u_new)
            del u_prev, v_prev, g
            key = (v_pre.view(torch.int32) & 0x7FFFFFFF).view(T, C)
            th = torch.from_numpy(theta.astype(np.int64)).cuda().view(T, 1)
            want = ((key != 0) & (key.long() >= th)).flatten()
            del key
            sel = torch.cat([idx[coff[c]:coff[c] + cnt[c]].long() + c * C for c in range(T)])
            vsel = torch.cat([val[coff[c]:coff[c] + cnt[c]] for c in range(T)])
            mask = torch.zeros(wl.n, dtype=torch.bool, device="cuda")
            mask[sel] = True
            assert torch.equal(mask, want)
            sent = torch.zeros_like(v_pre)
            sent[sel] = vsel
            assert torch.equal((sent + L.v[: wl.n]).view(torch.int32),
                               (v_pre + 0.0).view(torch.int32))
            assert bool((L.u[: wl.n][mask].view(torch.int32) == 0).all())
            assert torch.equal(L.u[: wl.n][~mask].view(torch.int32),
                               u_new[~mask].view(torch.int32))
            del sent, mask, want, sel, vsel, v_pre, u_new
        say(f"flat1b sampled step {t}: decode")
        dense = torch.zeros(wl.n, dtype=torch.float32, device="cuda")
        dgc.decode_accumulate(learners[0], [(L.runs, L.vals, L.entries) for L in learners],
                              dense)
        torch.cuda.synchronize()
        assert learners[0].status() == dgc.DGC_OK
        for c in SAMPLED:
            want_d = np.zeros(C, np.float32)
            for w in range(len(learners)):
                r, v_ = o_streams[w][c]
                assert oracle.decode_accumulate(r, v_, want_d) == 0
            got = dense[c * C:(c + 1) * C].cpu().numpy()
            assert np.array_equal(f32_bits(got), f32_bits(want_d)), (t, c)

        # the fresh sum the benchmark times: dgc_decode_sum into a buffer of NaNs
        fresh = torch.full_like(dense, float("nan"))
        dgc.decode_sum(learners[0], [(L.runs, L.vals, L.entries) for L in learners], fresh)
        torch.cuda.synchronize()
        assert learners[0].status() == dgc.DGC_OK
        assert torch.equal(fresh.view(torch.int32), dense.view(torch.int32)), t
        del fresh
        del dense
