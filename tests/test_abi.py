"""The C-ABI library: it loads, exports every entry point that include/dgc.h
declares, and its host-side argument checks return the documented codes
without touching a GPU."""

import ctypes
import os
import re
import subprocess
from fractions import Fraction

import numpy as np
import pytest

from conftest import ROOT

from sparsified_gradient_compression_amd import dgc

HEADER = os.path.join(ROOT, "include", "dgc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dgc_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 20, names
    L = dgc.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", dgc.lib_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (dgc_\w+)", out))
    assert set(names) <= exported


def test_binding_constants_match_the_header():
    """Every integer #define of include/dgc.h that the binding names holds
    the header's value, and the binding names every DGC_OPT_, DGC_TIMER_
    and error code."""
    defs = dict((m.group(1), int(m.group(2))) for m in re.finditer(
        r"#define\s+(DGC_\w+)\s+\(?(-?\d+)\)?", open(HEADER).read()))
    assert len(defs) >= 15, defs
    for name, value in defs.items():
        if name.startswith(("DGC_OPT_", "DGC_TIMER_", "DGC_E", "DGC_OK")):
            assert getattr(dgc, name) == value, name
        elif hasattr(dgc, name):
            assert getattr(dgc, name) == value, name


def test_error_strings():
    assert dgc.dgc_error_string(0) == "ok"
    assert dgc.dgc_error_string(-1) == "invalid argument"
    assert dgc.dgc_error_string(-4) == "corrupt stream"
    assert dgc.dgc_error_string(123) == "unknown error"


def test_workspace_bytes_validation():
    L = dgc.lib()
    out = ctypes.c_size_t(0)

    def call(sizes, kmax):
        s = np.asarray(sizes, np.int64)
        k = np.asarray(kmax, np.int64)
        return L.dgc_workspace_bytes(len(s), s.ctypes.data, k.ctypes.data,
                                     ctypes.byref(out))

    assert call([10, 20], [1, 1]) == 0 and out.value > 0
    assert call([10], [11]) == dgc.DGC_EINVAL       # k_max > n
    assert call([10], [-1]) == dgc.DGC_EINVAL
    assert call([1 << 32], [1]) == dgc.DGC_EINVAL   # local indices are 32-bit
    assert call([-5], [0]) == dgc.DGC_EINVAL
    assert L.dgc_workspace_bytes(0, None, None, ctypes.byref(out)) == dgc.DGC_EINVAL
    assert call([0, 7], [0, 7]) == 0                # empty tensors are allowed


def test_workspace_grows_with_k_max():
    small = dgc.dgc_workspace_bytes([1 << 24] * 4, [16778] * 4)
    big = dgc.dgc_workspace_bytes([1 << 24] * 4, [1 << 22] * 4)
    assert big > small


def test_init_and_calls_reject_bad_arguments_before_any_launch():
    L = dgc.lib()
    st = ctypes.c_void_p()
    s = np.array([100], np.int64)
    k = np.array([1], np.int64)
    # no workspace
    assert L.dgc_init_state(ctypes.byref(st), 1, s.ctypes.data, k.ctypes.data,
                            0.9, 256, 256, None, 0, None) == dgc.DGC_EINVAL
    # misaligned workspace
    assert L.dgc_init_state(ctypes.byref(st), 1, s.ctypes.data, k.ctypes.data,
                            0.9, 256, 256, 4096 + 8, 1 << 20, None) == dgc.DGC_EINVAL
    # workspace too small
    assert L.dgc_init_state(ctypes.byref(st), 1, s.ctypes.data, k.ctypes.data,
                            0.9, 256, 256, 4096, 16, None) == dgc.DGC_ECAPACITY
    # misaligned u
    assert L.dgc_init_state(ctypes.byref(st), 1, s.ctypes.data, k.ctypes.data,
                            0.9, 260, 256, 4096, 1 << 30, None) == dgc.DGC_EINVAL
    assert st.value is None
    assert L.dgc_compress(None, None, None, 0.0, None, None, None, None, None) == dgc.DGC_EINVAL
    assert L.dgc_encode(None, None, None, None, None, None, None, None) == dgc.DGC_EINVAL
    assert L.dgc_compress_binlocal(None, None, None, None, 0.0, None, None, None, None,
                                   None, None, None) == dgc.DGC_EINVAL
    assert L.dgc_encode_counts(None, None, None, None, None, None, None, None,
                               None) == dgc.DGC_EINVAL
    assert L.dgc_compress_sampled(None, None, None, None, 0.0, None, None, None, None,
                                  None, None, None) == dgc.DGC_EINVAL
    assert L.dgc_compress_shared(None, None, None, None, 0.0, None, None, None,
                                 None) == dgc.DGC_EINVAL
    assert L.dgc_compress_hier(None, None, None, 0.0, None, None, None, None, None,
                               None) == dgc.DGC_EINVAL
    assert L.dgc_shared_sum(None, 1, None, None, None, None, None, None) == dgc.DGC_EINVAL
    assert L.dgc_decode_accumulate(None, 1, None, None, None, None, None) == dgc.DGC_EINVAL
    assert L.dgc_decode_sum(None, 1, None, None, None, None, None) == dgc.DGC_EINVAL
    assert L.dgc_decode_sum(None, 0, None, None, None, None, None) == dgc.DGC_EINVAL
    assert L.dgc_get_status(None) == dgc.DGC_EINVAL
    assert L.dgc_set_option(None, 1, 0) == dgc.DGC_EINVAL
    assert L.dgc_set_fused_event(None, None) == dgc.DGC_EINVAL
    L.dgc_destroy_state(None)


def test_k_schedule_through_the_c_symbol():
    """dgc_k_for_density (DGC review, "Proposed method", warm-up): exact
    ceil(n * num / den) in the library, called through the raw C symbol."""
    L = dgc.lib()
    assert L.dgc_k_for_density(350_000_000, 1, 1000) == 350_000
    assert L.dgc_k_for_density(350_000_000, 1, 4) == 87_500_000
    assert L.dgc_k_for_density(350_000_000, 1, 250) == 1_400_000
    assert L.dgc_k_for_density(1 << 20, 1, 1000) == 1049
    assert L.dgc_k_for_density(1 << 24, 1, 1000) == 16778
    assert L.dgc_k_for_density(64, 1, 1000) == 1
    assert L.dgc_k_for_density(0, 1, 1000) == 0
    assert L.dgc_k_for_density(7, 0, 5) == 0
    assert L.dgc_k_for_density(7, 5, 5) == 7
    # the 128-bit product: n * num overflows int64 here
    n, num, den = (1 << 62) + 3, (1 << 40) - 1, 1 << 40
    assert L.dgc_k_for_density(n, num, den) == -(-n * num // den)
    for bad in ((-1, 1, 2), (5, 1, 0), (5, -1, 2), (5, 3, 2)):
        assert L.dgc_k_for_density(*bad) == dgc.DGC_EINVAL, bad


def test_k_schedule_binding_is_exact():
    assert dgc.k_for_density(350_000_000, Fraction(1, 1000)) == 350_000
    assert dgc.k_for_density(350_000_000, (1, 1000)) == 350_000
    assert dgc.k_for_density(1 << 20, Fraction(1, 1000)) == 1049
    assert dgc.k_for_density(64, Fraction(1, 1000)) == 1
    assert dgc.k_for_density(0, Fraction(1, 1000)) == 0
    assert dgc.k_for_density(10, 1) == 10
    for n in range(1, 3000, 7):
        for d in (Fraction(1, 4), Fraction(1, 250), Fraction(3, 7)):
            want = -(-n * d.numerator // d.denominator)
            assert dgc.k_for_density(n, d) == want


def test_k_schedule_refuses_binary_floats():
    """1 / 1000 in binary64 is slightly above 1/1000, so a float density
    would give ceil(350e6 * 0.001) = 350001; the binding refuses it."""
    for bad in (1 / 1000, 0.25, np.float32(0.5), np.float64(0.001)):
        with pytest.raises(TypeError):
            dgc.k_for_density(350_000_000, bad)
    with pytest.raises(TypeError):
        dgc.k_for_density(100, (1.0, 1000))
    with pytest.raises(TypeError):
        dgc.k_for_density(100, "1/1000")
    with pytest.raises(dgc.DGCError):
        dgc.k_for_density(100, Fraction(3, 2))


def test_build_flags_keep_ieee_binary32():
    from sparsified_gradient_compression_amd import build
    flags = " ".join(build.HIPCC_FLAGS)
    assert "-ffp-contract=off" in flags
    assert "-fno-gpu-flush-denormals-to-zero" in flags
    assert "-packed-fp32-ops" in flags
    assert "gfx950" in flags


def test_bin_index_by_multiply_high_is_exact():
    """The bin-local kernels find the bin of offset e (< 1024) inside a piece
    as (e * ceil(2^32 / L)) >> 32 (e itself for L = 1); that equals e // L
    for every bin length the library accepts."""
    e = np.arange(1024, dtype=np.uint64)
    for L in range(2, dgc.DGC_MAX_BIN + 1):
        magic = np.uint64(((1 << 32) + L - 1) // L)
        assert np.array_equal((e * magic) >> np.uint64(32), e // np.uint64(L)), L


def test_bin_local_pieces_hold_whole_bins():
    """Pieces of L * floor(1024 / L) elements: whole bins, never fewer than
    513 elements, so ceil(n / 513) pieces per tensor always suffice."""
    for L in range(1, dgc.DGC_MAX_BIN + 1):
        plen = L * (1024 // L)
        assert plen % L == 0 and 513 <= plen <= 1024
