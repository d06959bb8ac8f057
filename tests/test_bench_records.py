"""bench.py --records: one JSON line per (measured step, learner), with the
compress call's algorithmic bytes counted as the bench line counts them.
Host-side formatting only; the GPU measurement pass fills the rows."""

import json
from types import SimpleNamespace

import pytest


def test_records_lines(tmp_path):
    import bench
    wl = SimpleNamespace(name="toy", n=1000, sizes=[600, 400], learners=2, clip=1.0)
    rows = [{"step": 7, "gradient_step": 1, "learner": w, "k": 10, "sent": 10,
             "stream_entries": 13, "compress_ms": 0.002, "k_fused_ms": 0.001,
             "encode_ms": 0.0005, "decode_ms_all_learners": 0.003} for w in range(2)]
    path = tmp_path / "rec.jsonl"
    bench.write_records(str(path), wl, "topk", rows)
    bench.write_records(str(path), wl, "topk", rows[:1])  # appends
    lines = [json.loads(x) for x in path.read_text().splitlines()]
    assert [r["learner"] for r in lines] == [0, 1, 0]
    r = lines[0]
    # 24 B/elem with clipping (g, u, v read; u, v written; g re-read) + 16 B/entry
    assert r["compress_alg_bytes"] == 1000 * 24 + 16 * 10
    assert r["compress_GBps"] == pytest.approx(24160 / 2e-6 / 1e9, abs=0.1)
    assert r["compress_frac_of_peak"] == pytest.approx(24160 / 2e-6 / 1e9 / 8000, abs=1e-4)
    assert (r["workload"], r["selector"], r["elements"], r["tensors"]) == ("toy", "topk", 1000, 2)


def test_records_without_times(tmp_path):
    import bench
    wl = SimpleNamespace(name="toy", n=64, sizes=[64], learners=1, clip=0.0)
    rows = [{"step": 0, "gradient_step": 0, "learner": 0, "k": 4, "sent": 3,
             "stream_entries": None, "compress_ms": 0.0, "k_fused_ms": None,
             "encode_ms": None, "decode_ms_all_learners": None}]
    path = tmp_path / "rec.jsonl"
    bench.write_records(str(path), wl, "hier", rows)
    r = json.loads(path.read_text())
    assert r["compress_alg_bytes"] == 64 * 20 + 16 * 3
    assert r["compress_GBps"] is None and r["compress_frac_of_peak"] is None


def test_ranges_are_roctx_ranges_or_nothing():
    """--ranges wraps the step's calls in torch's range markers (roctx on
    ROCm; they need no GPU); without it, a context that does nothing."""
    import contextlib
    import bench
    off = SimpleNamespace(args=SimpleNamespace(ranges=False))
    assert isinstance(bench.Run.rng(off, "step 0"), contextlib.nullcontext)
    on = SimpleNamespace(args=SimpleNamespace(ranges=True))
    with bench.Run.rng(on, "step 0"):
        pass
