"""libdgc's host code (layout planning, argument checks) under AddressSanitizer
and UndefinedBehaviorSanitizer.  Only the host pass is instrumented; the
driver makes no GPU call, so it runs without a GPU."""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "sparsified_gradient_compression_amd", "csrc")


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_check"
    sanitize = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    cmd = (["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops"] + sanitize +
           ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, "dgc_api.hip"), os.path.join(ROOT, "tests", "host_check.cpp"),
            "-o", str(exe)])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-1000:], r.stderr[-3000:])
    assert "host check: ok" in r.stdout
