"""The committed rocprofv3 summaries under profiles/ match the kernels they
describe: each HBM traffic record carries a hash of its kernel sources, and
bench.py reports the record only while that hash matches; a stale record
would silently turn roofline.traffic into null."""

import json
import os

import pytest

from conftest import ROOT


@pytest.mark.parametrize("selector", ["topk", "binlocal", "sampled", "hier", "shared"])
def test_traffic_record_matches_current_kernel_sources(selector):
    import bench
    path, _ = bench.TRAFFIC[selector]
    rec = json.load(open(path))
    assert rec["kernel_source_sha"] == bench.kernel_source_sha(selector), (
        f"{os.path.basename(path)} was taken on other kernel sources: profile again")
    assert rec["n_elems"] == 1 << 30
    assert 1.0 <= rec["traffic_over_algorithmic"] < 1.1
    assert rec["copy_calibration"]["write_factor"] == pytest.approx(1.0, abs=0.01)


def test_profile_summaries_name_their_commands():
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not name.endswith(".md"):
            continue
        text = open(os.path.join(ROOT, "profiles", name)).read()
        assert "rocprofv3" in text and "bench.py" in text, name
        assert "_work" not in text, name
