"""Benchmark of the per-learner DGC compressor on one MI355X.

One step = the whole hot path over one batch of synthetic gradients: for each
of the W learners, dgc_compress (clip, momentum correction, exact top-k,
compaction, masking) and dgc_encode; then all W streams are decoded into a
fresh dense sum (dgc_decode_sum: every element written, none read, the same
bits as zeroing and dgc_decode_accumulate).  Inputs are resident in HBM
before the timed region; each step uses the next of the workload's gradient
steps, cycling.

Prints one JSON line.  value = gradient elements compressed per second (all
learners) over the K timed steps, wall clock; the timed region carries only
two HIP events per learner-step, around the element-wise pass (the dominant
kernel), whose average duration gives roofline.achieved, plus one event per
step boundary for the per-step median.  A separate, untimed measurement pass
with every library timer on gives the medians over steps x learners of the
compress, encode and decode times.  With the default workload (flat1b) and
selector, detail.workloads repeats the same measurement, bounded, on the
other four workloads (flat1m, resnet50, deepspeech, warmup350m).
cpu_baseline = the CPU oracle timed on a bounded sample of the headline
workload.

With --selector binlocal the step uses AdaComp's bin-local selector instead
of exact top-k (dgc_compress_binlocal + dgc_encode_counts, bins of
--bin-len entries, at most n_t / --cap-den entries delivered per tensor).
With --selector sampled it uses the sampled (approximate) threshold for the
same k as top-k (dgc_compress_sampled + dgc_encode_counts, at most 4 k per
tensor delivered) and reports how far the sent counts are from k.
With --selector hier it uses hierarchical thresholding for the same k:
the sampled threshold, then an exact select of k among its survivors when
more than k pass (dgc_compress_hier + dgc_encode_counts, at most k sent).
With --selector shared it uses shared-index compression (the ScaleComp
reading): the leader (step mod W) runs dgc_compress + dgc_encode, the other
learners dgc_compress_shared at its indices, and dgc_shared_sum adds the
value vectors in learner order into the fresh dense sum.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flat1b]
                    [--selector topk|binlocal|sampled|hier|shared] [--bin-len 512] [--cap-den 8]
"""

import argparse
import contextlib
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CSRC = os.path.join(ROOT, "sparsified_gradient_compression_amd", "csrc")
# committed counter summaries of the element-wise pass, per selector
TRAFFIC = {
    "topk": (os.path.join(ROOT, "profiles", "fused_flat1b_traffic.json"),
             ("dgc_device.hpp", "kernel_fused.hpp")),
    "binlocal": (os.path.join(ROOT, "profiles", "bl_fused_flat1b_traffic.json"),
                 ("dgc_device.hpp", "kernel_fused.hpp", "kernels_binlocal.hpp")),
    "sampled": (os.path.join(ROOT, "profiles", "sm_fused_flat1b_traffic.json"),
                ("dgc_device.hpp", "kernel_fused.hpp", "kernels_binlocal.hpp")),
    "hier": (os.path.join(ROOT, "profiles", "hier_fused_flat1b_traffic.json"),
             ("dgc_device.hpp", "kernel_fused.hpp")),
    "shared": (os.path.join(ROOT, "profiles", "sh_fused_flat1b_traffic.json"),
               ("dgc_device.hpp", "kernel_fused.hpp", "kernels_shared.hpp")),
}
# the other workloads measured after the headline: (name, timed steps)
OTHER_WORKLOADS = (("flat1m", 200), ("resnet50", 50), ("deepspeech", 20),
                   ("warmup350m", 10))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def file_sha16(path):
    h = hashlib.sha256()
    with open(path, "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_source_sha(selector="topk"):
    h = hashlib.sha256()
    for f in TRAFFIC[selector][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(n_elems, selector="topk"):
    """HBM bytes per launch of the element-wise pass from the committed
    rocprofv3 counter summary, if it was taken on the current kernel."""
    if selector not in TRAFFIC:
        return None
    try:
        with open(TRAFFIC[selector][0]) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_sha(selector):
        return None
    if rec.get("n_elems") != n_elems:
        return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="flat1b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip detail.workloads (the other four workloads)")
    ap.add_argument("--measure-steps", type=int, default=10,
                    help="steps of the untimed pass with every library timer on")
    ap.add_argument("--cpu-sample-chunks", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="cycle the oracle over the sample until this long")
    ap.add_argument("--grad-steps", type=int, default=0,
                    help="generate only this many gradient steps and cycle "
                         "over them (0: all of the workload's; for profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, run one plain device copy "
                         "of 1 GiB (for scaling hardware byte counters)")
    ap.add_argument("--pipeline", action="store_true",
                    help="run each learner on its own stream, starting once the "
                         "previous learner's element-wise pass is done")
    ap.add_argument("--select-grid", type=int, choices=(0, 1, 2), default=0,
                    help="DGC_OPT_SELECT_GRID for dgc_compress and dgc_compress_hier: 0 "
                         "automatic, 1 a workgroup "
                         "per tensor, 2 the spread passes")
    ap.add_argument("--encode-path", type=int, choices=(0, 1, 2), default=0,
                    help="DGC_OPT_ENCODE_PATH: 0 automatic, 1 a workgroup per "
                         "tensor, 2 the tiled passes")
    ap.add_argument("--decode-path", type=int, choices=(0, 1, 2, 3), default=0,
                    help="DGC_OPT_DECODE_PATH: 0 automatic, 1 each stream on its own "
                         "(tiled passes), 2 merged, 3 each stream on its own (a "
                         "workgroup per tensor)")
    ap.add_argument("--timers", choices=("fused", "off"), default="fused",
                    help="library timers in the timed region: the element-wise "
                         "pass only (default), or none (then roofline is null)")
    ap.add_argument("--selector", choices=("topk", "binlocal", "sampled", "hier", "shared"),
                    default="topk",
                    help="exact per-tensor top-k (DGC), AdaComp's bin-local rule, the "
                         "sampled threshold, the sampled threshold with an exact "
                         "top-k among its survivors, or shared-index compression "
                         "(ScaleComp)")
    ap.add_argument("--ranges", action="store_true",
                    help="roctx ranges around each step, learner call and decode "
                         "(for rocprofv3 --marker-trace); off by default")
    ap.add_argument("--records", default="",
                    help="write one JSON line per (measured step, learner) to this "
                         "file: k, sent entries, stream entries, times, algorithmic "
                         "bytes and rates")
    ap.add_argument("--bin-len", type=int, default=512,
                    help="bin length for --selector binlocal (1..1024)")
    ap.add_argument("--cap-den", type=int, default=8,
                    help="--selector binlocal delivers at most n_t // cap_den "
                         "entries per tensor")
    return ap.parse_args()


def cpu_baseline_binlocal(wl, host_samples, n_chunks, seconds, bin_len, cap_den):
    """As cpu_baseline, with the oracle's bin-local selector."""
    import oracle
    sizes = np.array(wl.sizes[:n_chunks], np.int64)
    Ls = np.full(len(sizes), bin_len, np.int64)
    caps = sizes // cap_den
    n = int(sizes.sum())
    u = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    dense = np.zeros(n, np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    coff = np.concatenate([[0], np.cumsum(caps)])
    t0 = time.perf_counter()
    steps = 0
    for cycle in range(4):
        for g in host_samples:
            idx, val, cnt, _, _, _ = oracle.binlocal_step(sizes, Ls, caps, g, u, v,
                                                          wl.momentum, wl.clip)
            dense[:] = 0
            for t in range(len(sizes)):
                a = coff[t]
                r, vv = oracle.encode(idx[a:a + cnt[t]], val[a:a + cnt[t]])
                oracle.decode_accumulate(r, vv, dense[offs[t]:offs[t + 1]])
            steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(n * steps / dt / 1e9, 4),
        "unit": "G elem/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"learner 0, {steps} steps, first {n_chunks} of "
                   f"{len(wl.sizes)} tensors ({n} elements): clip over the sample, "
                   f"momentum, bin-local select (bins of {bin_len}), mask, encode, "
                   f"decode; {dt:.1f} s"),
    }


def cpu_baseline_sampled(wl, host_samples, n_chunks, seconds):
    """As cpu_baseline, with the oracle's sampled-threshold selector."""
    import oracle
    sizes = np.array(wl.sizes[:n_chunks], np.int64)
    d = wl.densities[0]
    k = np.array([oracle.k_for_density(int(s), d.numerator, d.denominator) for s in sizes])
    caps = 4 * k
    n = int(sizes.sum())
    u = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    dense = np.zeros(n, np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    coff = np.concatenate([[0], np.cumsum(caps)])
    t0 = time.perf_counter()
    steps = 0
    for cycle in range(4):
        for g in host_samples:
            idx, val, cnt, _, _, _, _ = oracle.sampled_step(sizes, k, caps, g, u, v,
                                                            wl.momentum, wl.clip)
            dense[:] = 0
            for t in range(len(sizes)):
                a = coff[t]
                r, vv = oracle.encode(idx[a:a + cnt[t]], val[a:a + cnt[t]])
                oracle.decode_accumulate(r, vv, dense[offs[t]:offs[t + 1]])
            steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(n * steps / dt / 1e9, 4),
        "unit": "G elem/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"learner 0, {steps} steps, first {n_chunks} of "
                   f"{len(wl.sizes)} tensors ({n} elements): clip over the sample, "
                   "momentum, sampled threshold, mask, encode, decode; "
                   f"{dt:.1f} s"),
    }


def cpu_baseline_hier(wl, host_samples, n_chunks, seconds):
    """As cpu_baseline, with the oracle's hierarchical selector."""
    import oracle
    sizes = np.array(wl.sizes[:n_chunks], np.int64)
    d = wl.densities[0]
    k = np.array([oracle.k_for_density(int(s), d.numerator, d.denominator) for s in sizes])
    n = int(sizes.sum())
    u = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    dense = np.zeros(n, np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    koff = np.concatenate([[0], np.cumsum(k)])
    t0 = time.perf_counter()
    steps = 0
    for cycle in range(4):
        for g in host_samples:
            idx, val, cnt, _, _, _, _ = oracle.hier_step(sizes, k, g, u, v, wl.momentum,
                                                         wl.clip)
            dense[:] = 0
            for t in range(len(sizes)):
                a = koff[t]
                r, vv = oracle.encode(idx[a:a + cnt[t]], val[a:a + cnt[t]])
                oracle.decode_accumulate(r, vv, dense[offs[t]:offs[t + 1]])
            steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(n * steps / dt / 1e9, 4),
        "unit": "G elem/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"learner 0, {steps} steps, first {n_chunks} of "
                   f"{len(wl.sizes)} tensors ({n} elements): clip over the sample, "
                   "momentum, sampled threshold, exact select among its survivors, "
                   f"mask, encode, decode; {dt:.1f} s"),
    }


def cpu_baseline_shared(wl, host_samples, n_chunks, seconds):
    """As cpu_baseline, with shared-index compression: per gradient step the
    leader's exact top-k, the other learners' gather and mask at its set
    (each with its own state, all fed learner 0's sample gradient), the
    learner-order sum and the dense scatter."""
    import oracle
    sizes = np.array(wl.sizes[:n_chunks], np.int64)
    d = wl.densities[0]
    k = np.array([oracle.k_for_density(int(s), d.numerator, d.denominator) for s in sizes])
    n = int(sizes.sum())
    Wn = wl.learners
    us = [np.zeros(n, np.float32) for _ in range(Wn)]
    vs = [np.zeros(n, np.float32) for _ in range(Wn)]
    dense = np.zeros(n, np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    koff = np.concatenate([[0], np.cumsum(k)])
    t0 = time.perf_counter()
    steps = 0
    for cycle in range(4):
        for g in host_samples:
            g = g[:n]
            lead = steps % Wn
            idx, lval, _, _ = oracle.step(sizes, k, g, us[lead], vs[lead], wl.momentum,
                                          wl.clip)
            vals = []
            for w in range(Wn):
                if w == lead:
                    vals.append(lval)
                else:
                    vals.append(oracle.shared_step(sizes, k, idx, g, us[w], vs[w],
                                                   wl.momentum, wl.clip)[0])
            ssum = oracle.shared_sum(vals)
            dense[:] = 0
            for t in range(len(sizes)):
                dense[offs[t] + idx[koff[t]:koff[t + 1]].astype(np.int64)] = \
                    ssum[koff[t]:koff[t + 1]]
            steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(n * Wn * steps / dt / 1e9, 4),
        "unit": "G elem/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"{Wn} learners fed learner 0's gradients, {steps} steps, first "
                   f"{n_chunks} of {len(wl.sizes)} tensors ({n} elements per learner): "
                   "clip, momentum, the leader's exact top-k, the others' gather and "
                   f"mask at its set, learner-order sum, dense scatter; {dt:.1f} s"),
    }


def cpu_baseline(wl, host_samples, n_chunks, seconds):
    """The oracle as it stands on the first n_chunks tensors of learner 0:
    compress + encode + decode per gradient step, cycling over the steps
    (state carried along) until `seconds` have passed, at most 4 cycles."""
    import oracle
    sizes = np.array(wl.sizes[:n_chunks], np.int64)
    k = np.array([oracle.k_for_density(int(s), wl.densities[0].numerator,
                                       wl.densities[0].denominator) for s in sizes])
    n = int(sizes.sum())
    u = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    dense = np.zeros(n, np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)])
    koff = np.concatenate([[0], np.cumsum(k)])
    t0 = time.perf_counter()
    steps = 0
    for cycle in range(4):
        for g in host_samples:
            idx, val, _, _ = oracle.step(sizes, k, g, u, v, wl.momentum, wl.clip)
            dense[:] = 0
            for t in range(len(sizes)):
                r, vv = oracle.encode(idx[koff[t]:koff[t + 1]], val[koff[t]:koff[t + 1]])
                oracle.decode_accumulate(r, vv, dense[offs[t]:offs[t + 1]])
            steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    elems = n * steps
    return {
        "value": round(elems / dt / 1e9, 4),
        "unit": "G elem/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"learner 0, {steps} steps, first {n_chunks} of "
                   f"{len(wl.sizes)} tensors ({n} elements): clip over the sample, "
                   "momentum, exact top-k, mask, encode, decode; "
                   f"{dt:.1f} s"),
        "single_thread": single_thread(wl, host_samples[0][:wl.sizes[0]], k[:1]),
    }


def single_thread(wl, g, k):
    """The oracle on one thread: one learner-step of the first tensor."""
    import oracle
    cores = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        n = g.size
        u = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
        t0 = time.perf_counter()
        idx, val, _, _ = oracle.step(np.array([n], np.int64), np.array(k), g, u, v,
                                     wl.momentum, wl.clip)
        r, vv = oracle.encode(idx, val)
        dense = np.zeros(n, np.float32)
        oracle.decode_accumulate(r, vv, dense)
        dt = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(n / dt / 1e9, 4), "unit": "G elem/s", "cores": 1,
            "sample": f"one step of the first tensor ({n} elements), {dt:.2f} s"}


def med(xs):
    return round(float(statistics.median(xs)), 4) if xs else None


class Run:
    """One workload and selector on the GPU: every (learner, step) gradient
    resident in HBM, one Learner per simulated learner, and the dense sum."""

    def __init__(self, wl, selector, args, gsteps, host_sample_chunks=0):
        import torch
        from sparsified_gradient_compression_amd import dgc
        from sparsified_gradient_compression_amd import workloads as W
        self.dgc = dgc
        self.wl = wl
        self.selector = selector
        self.args = args
        T = len(wl.sizes)
        self.T = T
        self.binlocal = selector == "binlocal"
        self.sampled = selector == "sampled"
        self.hier = selector == "hier"
        self.shared = selector == "shared"
        if self.binlocal:
            self.bins = [args.bin_len] * T
            self.caps = [s // args.cap_den for s in wl.sizes]
            self.ks = [self.caps]  # the delivery capacity takes k's place
            kmax = self.caps
        else:
            self.ks = [[dgc.k_for_density(s, d) for s in wl.sizes] for d in wl.densities]
            kmax = [max(k[t] for k in self.ks) for t in range(T)]
            if self.sampled:
                # deliver at most 4 k per tensor, following each step's k
                self.caps_by_step = [[min(s, 4 * kk) for s, kk in zip(wl.sizes, k)]
                                     for k in self.ks]
                kmax = [max(c[t] for c in self.caps_by_step) for t in range(T)]
        self.gsteps = gsteps
        n = wl.n
        self.grads = {}
        self.host_samples = []
        g_host = np.empty(n, np.float32)
        n_sample = sum(wl.sizes[:host_sample_chunks])
        for t in range(gsteps):
            for w in range(wl.learners):
                t0 = time.perf_counter()
                W.gradient(wl, w, t, out=g_host)
                self.grads[(w, t)] = torch.from_numpy(g_host).cuda()
                if w == 0 and n_sample:
                    self.host_samples.append(g_host[:n_sample].copy())
                if n >= (1 << 26):
                    log(f"{wl.name}: gradient learner {w} step {t}: "
                        f"{time.perf_counter() - t0:.1f} s")
        del g_host
        torch.cuda.synchronize()
        self.learners = [dgc.Learner(list(wl.sizes), kmax, wl.momentum)
                         for _ in range(wl.learners)]
        for L in self.learners:
            L.set_option(dgc.DGC_OPT_SELECT_GRID, args.select_grid)
            L.set_option(dgc.DGC_OPT_ENCODE_PATH, args.encode_path)
            L.set_option(dgc.DGC_OPT_DECODE_PATH, args.decode_path)
        self.dense = torch.zeros(n, dtype=torch.float32, device="cuda")
        if self.shared:
            self.out_sum = torch.empty(max(int(sum(kmax)), 1), dtype=torch.float32,
                                       device="cuda")
        self.main = torch.cuda.current_stream()
        self.pipeline = args.pipeline and selector == "topk"
        if self.pipeline:
            # One stream per learner.  Learner w+1 starts once learner w's
            # element-wise pass is done (event recorded by the library), so
            # its clip norm and element-wise pass overlap learner w's short
            # selection and encode kernels, and no two element-wise passes
            # overlap.
            self.streams = [torch.cuda.Stream() for _ in self.learners]
            self.fused_ev = [torch.cuda.Event() for _ in self.learners]
            for L, ev in zip(self.learners, self.fused_ev):
                L.set_fused_event(ev)

    def k_of_step(self, s):
        return self.ks[(s % self.gsteps) % len(self.ks)]

    def rng(self, name):
        """A roctx range (torch's markers map to roctx on ROCm) with
        --ranges, else nothing: rocprofv3 --marker-trace then shows each
        step, learner call and decode on the kernel timeline."""
        if not self.args.ranges:
            return contextlib.nullcontext()
        import torch
        return torch.cuda.nvtx.range(name)

    def step(self, s):
        """Enqueue step s: every learner's compress + encode, then the
        learners' fresh dense sum."""
        with self.rng(f"step {s}"):
            self._step(s)

    def _step(self, s):
        dgc, args, learners = self.dgc, self.args, self.learners
        t = s % self.gsteps
        k = self.ks[t % len(self.ks)]
        streams_of = lambda: [(L.runs, L.vals, L.entries) for L in learners]  # noqa: E731
        if self.shared:
            # the leader (step mod W) selects and encodes its index set (the
            # set's broadcast, in the pages' run-length format); the others
            # send and mask at it; the value vectors are summed in learner
            # order into the fresh dense sum
            lead = s % len(learners)
            Ld = learners[lead]
            K = int(sum(k))
            with self.rng(f"learner {lead} leader"):
                Ld.compress(self.grads[(lead, t)], k, self.wl.clip)
                Ld.encode(k)
            for w, L in enumerate(learners):
                if w != lead:
                    with self.rng(f"learner {w} shared"):
                        L.compress_shared(self.grads[(w, t)], k, Ld.idx[:K], self.wl.clip)
            with self.rng("shared sum"):
                dgc.shared_sum(learners[0], [L.val[:K] for L in learners], k, Ld.idx[:K],
                               self.out_sum, self.dense)
            return
        if self.hier:
            for w, L in enumerate(learners):
                with self.rng(f"learner {w}"):
                    L.compress_hier(self.grads[(w, t)], k, self.wl.clip)
                    L.encode_counts(k)
            with self.rng("decode"):
                dgc.decode_sum(learners[0], streams_of(), self.dense)
            return
        if self.binlocal or self.sampled:
            step_caps = self.caps if self.binlocal else self.caps_by_step[t % len(self.ks)]
            for w, L in enumerate(learners):
                with self.rng(f"learner {w}"):
                    if self.binlocal:
                        L.compress_binlocal(self.grads[(w, t)], self.bins, step_caps,
                                            self.wl.clip)
                    else:
                        L.compress_sampled(self.grads[(w, t)], k, step_caps, self.wl.clip)
                    L.encode_counts(step_caps)
            with self.rng("decode"):
                dgc.decode_sum(learners[0], streams_of(), self.dense)
            return
        if not self.pipeline:
            for w, L in enumerate(learners):
                with self.rng(f"learner {w}"):
                    L.compress(self.grads[(w, t)], k, self.wl.clip)
                    L.encode(k)
            with self.rng("decode"):
                dgc.decode_sum(learners[0], streams_of(), self.dense)
            return
        import torch
        for w, L in enumerate(learners):
            st = self.streams[w]
            if w == 0:
                st.wait_stream(self.main)  # the previous step's decode is done
            else:
                st.wait_event(self.fused_ev[w - 1])
            with torch.cuda.stream(st):
                L.compress(self.grads[(w, t)], k, self.wl.clip, stream=st)
                L.encode(k, stream=st)
        for st in self.streams:
            self.main.wait_stream(st)
        dgc.decode_sum(learners[0], streams_of(), self.dense, stream=self.main)

    def set_timing(self, mode):
        for L in self.learners:
            L.set_option(self.dgc.DGC_OPT_KERNEL_TIMING, mode)

    def drain_timers(self):
        for L in self.learners:
            for tm in range(4):
                L.kernel_time(tm)

    def check(self):
        for L in self.learners:
            assert L.status() == self.dgc.DGC_OK

    def timed(self, first, steps, timers):
        """Steps [first, first + steps) bracketed by synchronisations; returns
        (wall seconds, per-step ms from events on the main stream, average
        element-wise pass ms or None)."""
        import torch
        self.drain_timers()
        self.set_timing(2 if timers == "fused" else 0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            self.step(first + i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        fused = None
        if timers == "fused":
            tot, cnt = 0.0, 0
            for L in self.learners:
                a, b = L.kernel_time(self.dgc.DGC_TIMER_FUSED)
                tot, cnt = tot + a, cnt + b
            fused = tot / max(cnt, 1)
        self.set_timing(0)
        self.check()
        return elapsed, step_ms, fused

    def measure(self, first, steps):
        """Untimed passes over the same steps, the library's timers read
        after each step.  The first brackets each call (compress, encode,
        decode); the second only the element-wise pass, since events inside a
        compress call would add their own overhead to it.  Per (step,
        learner) compress and element-wise ms, per step encode (mean over
        learners) and decode ms.  Returns lists and the k of each measured
        step."""
        dgc = self.dgc
        self.drain_timers()
        rec = {"compress": [], "fused": [], "encode": [], "decode": [], "k": [], "rows": []}
        self.set_timing(3)
        for i in range(steps):
            self.step(first + i)
            k = self.k_of_step(first + i)
            rec["k"].append(k)
            enc, rows, dec = [], [], None
            for w, L in enumerate(self.learners):
                c, nc = L.kernel_time(dgc.DGC_TIMER_COMPRESS)
                e, ne = L.kernel_time(dgc.DGC_TIMER_ENCODE)
                d, nd = L.kernel_time(dgc.DGC_TIMER_DECODE)
                rec["compress"].append((i, c / max(nc, 1)))
                if ne:
                    enc.append(e / ne)
                if nd:
                    rec["decode"].append(d / nd)
                    dec = d / nd
                # per (step, learner): what left the learner and its times
                sent = (int(sum(k)) if self.selector in ("topk", "shared")
                        else int(L.count.sum()))
                rows.append({"step": first + i, "gradient_step": (first + i) % self.gsteps,
                             "learner": w, "k": int(sum(k)), "sent": sent,
                             "stream_entries": int(L.entries.sum()) if ne else None,
                             "compress_ms": round(c / max(nc, 1), 5),
                             "k_fused_ms": None,
                             "encode_ms": round(e / ne, 5) if ne else None})
            for r in rows:
                r["decode_ms_all_learners"] = round(dec, 5) if dec is not None else None
            rec["rows"].extend(rows)
            if enc:
                rec["encode"].append(sum(enc) / len(enc))
        self.set_timing(2)
        for i in range(steps):
            self.step(first + i)
            for w, L in enumerate(self.learners):
                f, nf = L.kernel_time(dgc.DGC_TIMER_FUSED)
                if nf:
                    rec["fused"].append((i, f / nf))
                    rec["rows"][i * len(self.learners) + w]["k_fused_ms"] = round(f / nf, 5)
        self.set_timing(0)
        self.check()
        return rec

    def close(self):
        import torch
        for L in self.learners:
            L.close()
        self.learners = []
        self.grads = {}
        self.dense = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def compress_alg_bytes(wl, k):
    """Algorithmic bytes of one learner's compress at per-tensor k: read g,
    u, v and write u, v (20 B/elem), the norm's re-read of g (4 B/elem with
    clipping), the selected (index, value) written and u, v zeroed there
    (16 B per entry)."""
    clip = 1 if wl.clip > 0 else 0
    return wl.n * (20 + 4 * clip) + 16 * int(sum(k))


def write_records(path, wl, selector, rows):
    """One JSON line per (measured step, learner): the workload and selector,
    the step's k and what was sent, the library's timings, and the compress
    call's algorithmic bytes (counted as compress_alg_bytes counts them, at
    the entries sent) with its rate and fraction of 8 TB/s.  Appends."""
    with open(path, "a") as f:
        for r in rows:
            alg = compress_alg_bytes(wl, [r["sent"]])
            ms = r["compress_ms"]
            out = {"workload": wl.name, "selector": selector, "elements": wl.n,
                   "tensors": len(wl.sizes), "learners": wl.learners, "clip": wl.clip}
            out.update(r)
            out.update({"compress_alg_bytes": alg,
                        "compress_GBps": round(alg / (ms * 1e-3) / 1e9, 1) if ms else None,
                        "compress_frac_of_peak": (round(alg / (ms * 1e-3) / 1e9 /
                                                        HBM_PEAK_GBPS, 4) if ms else None),
                        "compress_G_elem_per_s": round(wl.n / (ms * 1e-3) / 1e9, 2) if ms else None})
            f.write(json.dumps(out) + "\n")


def workload_record(run, steps, warmup, measure_steps):
    """Whole-step throughput over `steps` timed steps, then the measurement
    pass; the per-density compress figures when k changes per step."""
    wl = run.wl
    for s in range(warmup):
        run.step(s)
    # no library timers in this timed region (the element-wise pass is
    # timed in the measurement pass): an event record between two kernels
    # delays the second by a few microseconds, a visible share of a small
    # workload's step
    elapsed, step_ms, fused = run.timed(warmup, steps, "off")
    rec = run.measure(warmup + steps, measure_steps)
    comp = [c for _, c in rec["compress"]]
    by_step = {}
    for (i, c) in rec["compress"]:
        by_step.setdefault(i, []).append(c)
    alg = [compress_alg_bytes(wl, rec["k"][i]) for i in sorted(by_step)]
    step_c = [statistics.mean(by_step[i]) for i in sorted(by_step)]
    frac = sum(alg) / (sum(step_c) * 1e-3) / 1e9 / HBM_PEAK_GBPS
    out = {
        "workload": wl.name,
        "elements_per_learner": wl.n,
        "tensors": len(wl.sizes),
        "learners": wl.learners,
        "steps_timed": steps,
        "whole_step_G_elem_per_s": round(wl.n * wl.learners * steps / elapsed / 1e9, 3),
        "step_ms_median": med(step_ms),
        "compress_ms_median": med(comp),
        "k_fused_ms_median": med([f for _, f in rec["fused"]]),
        "encode_ms_median": med(rec["encode"]),
        "decode_ms_median": med(rec["decode"]),
        "compress_alg_frac_of_peak": round(frac, 4),
    }
    if len(set(wl.densities)) > 1:
        per = {}
        for i, c in zip(sorted(by_step), step_c):
            d = str(wl.densities[(warmup + steps + i) % run.gsteps % len(run.ks)])
            per.setdefault(d, []).append((c, compress_alg_bytes(wl, rec["k"][i])))
        out["per_density"] = [
            {"density": d, "compress_ms": round(statistics.median(c for c, _ in v), 4),
             "frac_of_peak": round(v[0][1] / (statistics.median(c for c, _ in v) * 1e-3)
                                   / 1e9 / HBM_PEAK_GBPS, 4)}
            for d, v in per.items()]
        # the mean of the per-density fractions (each step weighted alike),
        # beside compress_alg_frac_of_peak (all bytes over all time)
        out["compress_alg_frac_of_peak_mean_over_densities"] = round(
            statistics.mean(x["frac_of_peak"] for x in out["per_density"]), 4)
    return out, elapsed, step_ms, fused, rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU exchange of the streams is not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparsified_gradient_compression_amd import dgc
    from sparsified_gradient_compression_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dgc.lib()
    torch.cuda.set_device(0)
    wl = W.get(args.workload)
    if args.records:
        open(args.records, "w").close()
    T = len(wl.sizes)
    n = wl.n
    gsteps = args.grad_steps if args.grad_steps > 0 else wl.steps
    run = Run(wl, args.selector, args, gsteps,
              0 if args.no_cpu_baseline else args.cpu_sample_chunks)
    for s in range(args.warmup):
        run.step(s)
    torch.cuda.synchronize()
    run.check()
    log("timed region")
    elapsed, step_ms, fused_ms = run.timed(args.warmup, args.steps, args.timers)
    if args.calibrate_copy:
        # a plain copy of known size: reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("measurement pass")
    first = args.warmup + args.steps
    rec = run.measure(first, args.measure_steps) if args.measure_steps > 0 else None
    if args.records and rec is not None:
        write_records(args.records, wl, args.selector, rec["rows"])
    learners = run.learners
    ks = run.ks
    elems = n * wl.learners * args.steps
    value = elems / elapsed / 1e9
    clip = 1 if wl.clip > 0 else 0
    last = first + max(args.measure_steps, 1) - 1
    if run.binlocal or run.sampled:
        # the last step's salient and delivered counts, all learners
        salient = int(sum(int(L.total.sum()) for L in learners)) // len(learners)
        delivered = int(sum(int(L.count.sum()) for L in learners)) // len(learners)
        truncated = int(sum(int((L.total > L.count).sum()) for L in learners))
        # read g, u, v; write u, v; 8 B per salient entry into its slot
        fused_bytes = 20 * n + 8 * salient
        # + norm re-read; + slot read, output write and u/v masking per entry
        pipeline_bytes = n * (20 + 4 * clip) + 8 * salient + 16 * delivered
        kernel_name = ("k_bl_fused (clip-scale + momentum correction + accumulation + "
                       + ("per-bin maxima + salient entries to slots)" if run.binlocal else
                          "entries at or above the sampled threshold to slots)"))
    elif run.shared:
        fused_bytes = 20 * n  # read g, u, v; write u, v (both passes)
        # per learner-step, the mean of one leader (top-k) and W - 1 followers
        # (the norm, 20 B/elem, the shared indices read, the values written)
        K = int(sum(ks[0]))
        follower = n * (20 + 4 * clip) + 8 * K
        pipeline_bytes = (compress_alg_bytes(wl, ks[0]) + (wl.learners - 1) * follower) \
            / wl.learners
        kernel_name = ("k_fused (leader) and k_sh_fused (the others: clip-scale + momentum "
                       "correction + accumulation + values at the shared indices, masked)")
    else:
        fused_bytes = 20 * n  # read g, u, v; write u, v
        pipeline_bytes = compress_alg_bytes(wl, ks[0])
        kernel_name = ("k_fused (clip-scale + momentum correction + accumulation + "
                       "candidate output)")
        if run.hier:
            kernel_name = kernel_name[:-1] + ": the first level's survivors)"
    roofline = None
    if fused_ms:
        achieved = fused_bytes / (fused_ms * 1e-3) / 1e9
        traffic = measured_traffic(n, args.selector)
        roofline = {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": fused_bytes,
            "avg_launch_ms": round(fused_ms, 4),
            # HBM bytes the counters saw per launch over this run's launch time
            "traffic_GBps": (round(traffic / (fused_ms * 1e-3) / 1e9, 1)
                             if traffic else None),
        }
    lib_path = dgc.lib_path()
    out = {
        "metric": "gradient elements compressed/sec (G elem/s) and % of MI355X peak HBM GB/s",
        "value": round(value, 3),
        "unit": "G elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "selector": args.selector,
            "elements_per_learner": n,
            "tensors": T,
            "learners": wl.learners,
            "clip": wl.clip,
            "momentum": wl.momentum,
            "gradient_steps": wl.steps,
        },
        "roofline": roofline,
        "detail": {
            "library": {"path": os.path.relpath(lib_path, ROOT),
                        "sha16": file_sha16(lib_path)},
            "timed_region_timers": ("two HIP events per learner-step around the "
                                    "element-wise pass" if args.timers == "fused"
                                    else "none"),
            "step_ms_median": med(step_ms),
            "step_ms_min_max": [round(min(step_ms), 4), round(max(step_ms), 4)],
        },
    }
    det = out["detail"]
    if rec is not None:
        comp = [c for _, c in rec["compress"]]
        comp_med = statistics.median(comp)
        det.update({
            "measured_steps": args.measure_steps,
            "compress_ms_median": med(comp),
            "k_fused_ms_median": med([f for _, f in rec["fused"]]),
            "encode_ms_median": med(rec["encode"]),
            "decode_ms_median": med(rec["decode"]),
            "compress_pipeline_alg_GBps": round(pipeline_bytes / (comp_med * 1e-3) / 1e9, 1),
            "compress_pipeline_frac_of_peak": round(
                pipeline_bytes / (comp_med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "compress_G_elem_per_s": round(n / (comp_med * 1e-3) / 1e9, 2),
        })
    if run.binlocal or run.sampled:
        if run.binlocal:
            out["config"].update({"bin_len": args.bin_len,
                                  "cap_per_tensor": f"n_t // {args.cap_den}"})
        else:
            klast = np.array(run.k_of_step(last))
            ratio = np.concatenate([L.total.cpu().numpy() / np.maximum(klast, 1)
                                    for L in learners])
            out["config"].update({"k_per_tensor": int(klast[0]) if len(set(klast)) == 1
                                  else "per tensor", "density": str(wl.densities[0]),
                                  "cap_per_tensor": "4 k"})
            det["sent_over_k_min_mean_max"] = [round(float(ratio.min()), 4),
                                               round(float(ratio.mean()), 4),
                                               round(float(ratio.max()), 4)]
        det.update({"salient_per_learner": salient,
                    "salient_fraction": round(salient / n, 5),
                    "delivered_per_learner": delivered,
                    "truncated_tensors": truncated})
    elif run.hier:
        klast = np.array(run.k_of_step(last))
        info = np.concatenate([L.select_info() for L in learners])
        kk = np.concatenate([klast] * len(learners))
        sent = np.concatenate([L.count.cpu().numpy() for L in learners])
        listed = info[:, 0] == 1
        out["config"].update({
            "k_per_tensor": int(klast[0]) if len(set(klast)) == 1 else "per tensor",
            "density": str(wl.densities[0])})
        det.update({
            "sent_over_k_min_mean_max": [round(float(x), 4) for x in (
                (sent / np.maximum(kk, 1)).min(), (sent / np.maximum(kk, 1)).mean(),
                (sent / np.maximum(kk, 1)).max())],
            "survivors_over_k_min_max": ([round(float((info[listed, 2] / kk[listed]).min()), 3),
                                         round(float((info[listed, 2] / kk[listed]).max()), 3)]
                                        if listed.any() else None),
            "sources_list_whole_select_dense": [
                int((listed & (info[:, 2] <= kk)).sum()), int((listed & (info[:, 2] > kk)).sum()),
                int((info[:, 0] == 2).sum())]})
    elif run.shared:
        out["config"].update({
            "k_per_tensor": ks[0][0] if len(set(ks[0])) == 1 else "per tensor",
            "density": str(wl.densities[0]),
            "leader": "step mod learners (exact top-k); the others at its indices"})
    else:
        path = [L.path_counts() for L in learners]
        info = np.concatenate([L.select_info() for L in learners])
        kk = np.array(list(run.k_of_step(last)) * len(learners))
        listed = info[:, 0] == 1
        cand_ratio = info[listed, 2] / np.maximum(kk[listed], 1)
        out["config"].update({
            "k_per_tensor": ks[0][0] if len(set(ks[0])) == 1 else "per tensor",
            "density": str(wl.densities[0])})
        det.update({
            "learner_pipelining": run.pipeline,
            "select_path_window_dense": [int(sum(p[0] for p in path)),
                                         int(sum(p[1] for p in path))],
            "overflow_tensors": int(info[:, 3].sum()),
            "window_candidates_over_k": ([round(float(cand_ratio.min()), 3),
                                          round(float(cand_ratio.max()), 3)]
                                         if cand_ratio.size else None)})
    host_samples = run.host_samples
    run.close()
    del run
    if (not args.no_workloads and args.workload == "flat1b" and args.selector == "topk"
            and not args.pipeline):
        det["workloads"] = []
        for name, steps in OTHER_WORKLOADS:
            log(f"workload {name}")
            owl = W.get(name)
            orun = Run(owl, "topk", args, owl.steps)
            r, _, _, _, orec = workload_record(orun, steps, owl.steps, 2 * owl.steps
                                               if owl.steps > 1 else 10)
            if args.records:
                write_records(args.records, owl, "topk", orec["rows"])
            orun.close()
            det["workloads"].append(r)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        if args.selector == "binlocal":
            out["cpu_baseline"] = cpu_baseline_binlocal(
                wl, host_samples, args.cpu_sample_chunks, args.cpu_seconds,
                args.bin_len, args.cap_den)
        elif args.selector == "sampled":
            out["cpu_baseline"] = cpu_baseline_sampled(
                wl, host_samples, args.cpu_sample_chunks, args.cpu_seconds)
        elif args.selector == "hier":
            out["cpu_baseline"] = cpu_baseline_hier(
                wl, host_samples, args.cpu_sample_chunks, args.cpu_seconds)
        elif args.selector == "shared":
            out["cpu_baseline"] = cpu_baseline_shared(
                wl, host_samples, min(args.cpu_sample_chunks, 16), args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(wl, host_samples, args.cpu_sample_chunks,
                                               args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
