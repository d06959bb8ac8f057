"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only, g++), plus Hypothesis-generated inputs against brute force."""

import os
import shutil
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from conftest import ROOT
from oracle import bruteforce as bf

ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "check"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(ORACLE, "check_driver.cpp"),
           os.path.join(ORACLE, "dgc_oracle.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "ok" in r.stdout


MAGS = st.sampled_from([0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 0.25, 1e-40, -1e-40, 3e38])


@settings(max_examples=300, deadline=None)
@given(st.lists(st.one_of(MAGS, st.floats(-1e3, 1e3, width=32)), min_size=1, max_size=300),
       st.data())
def test_select_against_full_sort_hypothesis(orc, xs, data):
    v0 = np.array(xs, np.float32)
    k = data.draw(st.integers(0, v0.size))
    v = v0.copy()
    idx, val = orc.select_mask(np.zeros_like(v), v, k)
    assert np.array_equal(idx, bf.topk_fullsort(v0, k))
    assert np.array_equal(val.view(np.uint32), v0[idx].view(np.uint32))


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 300000), st.data())
def test_encode_against_walk_hypothesis(orc, n, data):
    picks = data.draw(st.lists(st.integers(0, n - 1), max_size=40, unique=True))
    idx = np.array(sorted(picks), np.uint32)
    val = np.arange(1, idx.size + 1, dtype=np.float32)
    runs, vals = orc.encode(idx, val)
    r2, v2 = bf.encode_walk(n, idx, val)
    assert np.array_equal(runs, r2) and np.array_equal(vals, v2)
