"""ctypes binding of libdgc (include/dgc.h): the same entry points, with
torch tensors marshalled to device pointers.  No computation happens here;
every step of the compressor runs in the HIP kernels of libdgc.so, and the
binding refuses to run without that library.
"""

from __future__ import annotations

import ctypes
import os
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import build as _build

DGC_OK = 0
DGC_EINVAL = -1
DGC_ECAPACITY = -2
DGC_EHIP = -3
DGC_ECORRUPT = -4
DGC_OPT_SELECT_PATH = 1
DGC_OPT_KERNEL_TIMING = 2
DGC_OPT_DECODE_PATH = 3
DGC_OPT_SELECT_GRID = 4
DGC_OPT_ENCODE_PATH = 5
DGC_TIMER_FUSED = 0
DGC_TIMER_COMPRESS = 1
DGC_TIMER_ENCODE = 2
DGC_TIMER_DECODE = 3
DGC_MAX_BIN = 1024

_lib = None


class DGCError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {dgc_error_string(code)} ({code})")


def lib_path() -> str:
    """The library this binding loads: the in-tree build, always."""
    return _build.LIB


def lib() -> ctypes.CDLL:
    """Load libdgc.so.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m sparsified_gradient_compression_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    L.dgc_k_for_density.argtypes = [i64, i64, i64]
    L.dgc_k_for_density.restype = i64
    L.dgc_workspace_bytes.argtypes = [i32, P, P, ctypes.POINTER(ctypes.c_size_t)]
    L.dgc_workspace_bytes.restype = ctypes.c_int
    L.dgc_init_state.argtypes = [ctypes.POINTER(P), i32, P, P, ctypes.c_float,
                                 P, P, P, ctypes.c_size_t, P]
    L.dgc_init_state.restype = ctypes.c_int
    L.dgc_compress.argtypes = [P, P, P, ctypes.c_double, P, P, P, P, P]
    L.dgc_compress.restype = ctypes.c_int
    L.dgc_compress_binlocal.argtypes = [P, P, P, P, ctypes.c_double, P, P, P, P,
                                        P, P, P]
    L.dgc_compress_binlocal.restype = ctypes.c_int
    L.dgc_compress_sampled.argtypes = [P, P, P, P, ctypes.c_double, P, P, P, P,
                                       P, P, P]
    L.dgc_compress_sampled.restype = ctypes.c_int
    L.dgc_compress_hier.argtypes = [P, P, P, ctypes.c_double, P, P, P, P, P, P]
    L.dgc_compress_hier.restype = ctypes.c_int
    L.dgc_compress_shared.argtypes = [P, P, P, P, ctypes.c_double, P, P, P, P]
    L.dgc_compress_shared.restype = ctypes.c_int
    L.dgc_shared_sum.argtypes = [P, i32, P, P, P, P, P, P]
    L.dgc_shared_sum.restype = ctypes.c_int
    L.dgc_encode_counts.argtypes = [P, P, P, P, P, P, P, P, P]
    L.dgc_encode_counts.restype = ctypes.c_int
    L.dgc_stream_capacity.argtypes = [P, P]
    L.dgc_stream_capacity.restype = ctypes.c_int
    L.dgc_encode.argtypes = [P, P, P, P, P, P, P, P]
    L.dgc_encode.restype = ctypes.c_int
    L.dgc_decode_accumulate.argtypes = [P, i32, P, P, P, P, P]
    L.dgc_decode_accumulate.restype = ctypes.c_int
    L.dgc_decode_sum.argtypes = [P, i32, P, P, P, P, P]
    L.dgc_decode_sum.restype = ctypes.c_int
    L.dgc_get_status.argtypes = [P]
    L.dgc_get_status.restype = ctypes.c_int
    L.dgc_get_path_counts.argtypes = [P, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.dgc_get_path_counts.restype = ctypes.c_int
    L.dgc_get_select_info.argtypes = [P, P]
    L.dgc_get_select_info.restype = ctypes.c_int
    L.dgc_set_fused_event.argtypes = [P, P]
    L.dgc_set_fused_event.restype = ctypes.c_int
    L.dgc_set_option.argtypes = [P, i32, i64]
    L.dgc_set_option.restype = ctypes.c_int
    L.dgc_get_kernel_time.argtypes = [P, i32, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(i64)]
    L.dgc_get_kernel_time.restype = ctypes.c_int
    L.dgc_destroy_state.argtypes = [P]
    L.dgc_destroy_state.restype = None
    L.dgc_error_string.argtypes = [ctypes.c_int]
    L.dgc_error_string.restype = ctypes.c_char_p
    _lib = L
    return L


# ---------------------------------------------------------------- marshalling

def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _hp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dp(t) -> Optional[int]:
    """Device pointer of a torch tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str):
    if rc != DGC_OK:
        raise DGCError(rc, what)


# ---------------------------------------------------------------- entry points

def dgc_error_string(code: int) -> str:
    return lib().dgc_error_string(int(code)).decode()


def dgc_workspace_bytes(sizes: Sequence[int], k_max: Sequence[int]) -> int:
    s, km = _i64(sizes), _i64(k_max)
    out = ctypes.c_size_t(0)
    _check(lib().dgc_workspace_bytes(len(s), _hp(s), _hp(km), ctypes.byref(out)),
           "dgc_workspace_bytes")
    return int(out.value)


def dgc_init_state(sizes, k_max, momentum: float, u, v, workspace,
                   stream=None) -> ctypes.c_void_p:
    s, km = _i64(sizes), _i64(k_max)
    st = ctypes.c_void_p()
    _check(lib().dgc_init_state(ctypes.byref(st), len(s), _hp(s), _hp(km),
                                float(momentum), _dp(u), _dp(v), _dp(workspace),
                                workspace.numel() * workspace.element_size(),
                                _stream(stream)),
           "dgc_init_state")
    return st


def dgc_compress(st, g, k, clip: float, out_idx, out_val, out_norm=None,
                 out_scale=None, stream=None):
    kk = _i64(k)
    _check(lib().dgc_compress(st, _dp(g), _hp(kk), float(clip), _dp(out_idx),
                              _dp(out_val), _dp(out_norm), _dp(out_scale),
                              _stream(stream)),
           "dgc_compress")


def dgc_compress_binlocal(st, g, bin_len, cap, clip: float, out_idx, out_val,
                          out_count, out_total=None, out_norm=None,
                          out_scale=None, stream=None):
    bl, cc = _i64(bin_len), _i64(cap)
    _check(lib().dgc_compress_binlocal(st, _dp(g), _hp(bl), _hp(cc), float(clip),
                                       _dp(out_idx), _dp(out_val), _dp(out_count),
                                       _dp(out_total), _dp(out_norm),
                                       _dp(out_scale), _stream(stream)),
           "dgc_compress_binlocal")


def dgc_compress_hier(st, g, k, clip: float, out_idx, out_val, out_count,
                      out_norm=None, out_scale=None, stream=None):
    kk = _i64(k)
    _check(lib().dgc_compress_hier(st, _dp(g), _hp(kk), float(clip), _dp(out_idx),
                                   _dp(out_val), _dp(out_count), _dp(out_norm),
                                   _dp(out_scale), _stream(stream)),
           "dgc_compress_hier")


def dgc_compress_sampled(st, g, k, cap, clip: float, out_idx, out_val, out_count,
                         out_total=None, out_norm=None, out_scale=None, stream=None):
    kk, cc = _i64(k), _i64(cap)
    _check(lib().dgc_compress_sampled(st, _dp(g), _hp(kk), _hp(cc), float(clip),
                                      _dp(out_idx), _dp(out_val), _dp(out_count),
                                      _dp(out_total), _dp(out_norm), _dp(out_scale),
                                      _stream(stream)),
           "dgc_compress_sampled")


def dgc_compress_shared(st, g, k, shared_idx, clip: float, out_val, out_norm=None,
                        out_scale=None, stream=None):
    kk = _i64(k)
    _check(lib().dgc_compress_shared(st, _dp(g), _hp(kk), _dp(shared_idx), float(clip),
                                     _dp(out_val), _dp(out_norm), _dp(out_scale),
                                     _stream(stream)),
           "dgc_compress_shared")


def dgc_shared_sum(st, vals: Sequence, k, shared_idx, out_sum, dense=None, stream=None):
    kk = _i64(k)
    W = len(vals)
    Arr = ctypes.c_void_p * max(W, 1)
    vv = Arr(*[_dp(x) for x in vals])
    _check(lib().dgc_shared_sum(st, W, ctypes.cast(vv, ctypes.c_void_p), _hp(kk),
                                _dp(shared_idx), _dp(out_sum), _dp(dense),
                                _stream(stream)),
           "dgc_shared_sum")


def dgc_stream_capacity(st, n_tensors: int) -> np.ndarray:
    out = np.zeros(n_tensors + 1, np.int64)
    _check(lib().dgc_stream_capacity(st, _hp(out)), "dgc_stream_capacity")
    return out


def dgc_encode(st, k, idx, val, runs, vals, entries, stream=None):
    kk = _i64(k)
    _check(lib().dgc_encode(st, _hp(kk), _dp(idx), _dp(val), _dp(runs), _dp(vals),
                            _dp(entries), _stream(stream)),
           "dgc_encode")


def dgc_encode_counts(st, cap, count, idx, val, runs, vals, entries, stream=None):
    cc = _i64(cap)
    _check(lib().dgc_encode_counts(st, _hp(cc), _dp(count), _dp(idx), _dp(val),
                                   _dp(runs), _dp(vals), _dp(entries),
                                   _stream(stream)),
           "dgc_encode_counts")


def _decode(fn: str, st, runs: Sequence, vals: Sequence, entries: Sequence, dense,
            stream=None):
    W = len(runs)
    assert len(vals) == W and len(entries) == W
    Arr = ctypes.c_void_p * max(W, 1)
    r = Arr(*[_dp(x) for x in runs])
    vv = Arr(*[_dp(x) for x in vals])
    e = Arr(*[_dp(x) for x in entries])
    _check(getattr(lib(), fn)(st, W, ctypes.cast(r, ctypes.c_void_p),
                              ctypes.cast(vv, ctypes.c_void_p),
                              ctypes.cast(e, ctypes.c_void_p), _dp(dense),
                              _stream(stream)), fn)


def dgc_decode_accumulate(st, runs: Sequence, vals: Sequence, entries: Sequence,
                          dense, stream=None):
    _decode("dgc_decode_accumulate", st, runs, vals, entries, dense, stream)


def dgc_decode_sum(st, runs: Sequence, vals: Sequence, entries: Sequence, dense,
                   stream=None):
    _decode("dgc_decode_sum", st, runs, vals, entries, dense, stream)


def dgc_get_status(st) -> int:
    return int(lib().dgc_get_status(st))


def dgc_get_path_counts(st) -> Tuple[int, int]:
    nw, nd = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().dgc_get_path_counts(st, ctypes.byref(nw), ctypes.byref(nd)),
           "dgc_get_path_counts")
    return int(nw.value), int(nd.value)


def dgc_get_select_info(st, n_tensors: int) -> np.ndarray:
    """[n_tensors, 6] int64: path, window key, candidates, overflow, T, r."""
    out = np.zeros((n_tensors, 6), np.int64)
    _check(lib().dgc_get_select_info(st, _hp(out)), "dgc_get_select_info")
    return out


def dgc_set_fused_event(st, event):
    """event: a torch.cuda.Event (created here if needed), an int handle,
    or None to turn the hook off."""
    handle = None
    if event is not None:
        if isinstance(event, int):
            handle = event
        else:
            if not event.cuda_event:
                event.record()  # torch creates the HIP event lazily
            handle = event.cuda_event
    _check(lib().dgc_set_fused_event(st, handle), "dgc_set_fused_event")


def dgc_set_option(st, option: int, value: int):
    _check(lib().dgc_set_option(st, int(option), int(value)), "dgc_set_option")


def dgc_get_kernel_time(st, timer: int) -> Tuple[float, int]:
    ms, cnt = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().dgc_get_kernel_time(st, int(timer), ctypes.byref(ms),
                                     ctypes.byref(cnt)),
           "dgc_get_kernel_time")
    return float(ms.value), int(cnt.value)


def dgc_destroy_state(st):
    lib().dgc_destroy_state(st)


def _density_fraction(density) -> Tuple[int, int]:
    """(num, den) of an exact density: a Fraction, an int, or a (num, den)
    pair.  Binary floating point is refused: 1 / 1000 is not 1/1000."""
    if isinstance(density, tuple) and len(density) == 2:
        num, den = density
        if not all(isinstance(x, (int, np.integer)) and not isinstance(x, bool)
                   for x in (num, den)):
            raise TypeError("density (num, den) must be integers")
        return int(num), int(den)
    if isinstance(density, (float, np.floating)):
        raise TypeError("density must be exact (Fraction or (num, den)), not a "
                        f"float: {density!r} is not an exact fraction in binary")
    if isinstance(density, (Fraction, int, np.integer)) and not isinstance(density, bool):
        d = Fraction(density)
        return d.numerator, d.denominator
    raise TypeError(f"density must be a Fraction, an int or (num, den), not "
                    f"{type(density).__name__}")


def dgc_k_for_density(n: int, num: int, den: int) -> int:
    k = int(lib().dgc_k_for_density(int(n), int(num), int(den)))
    if k < 0:
        raise DGCError(k, "dgc_k_for_density")
    return k


def k_for_density(n: int, density) -> int:
    """Entries a tensor of n elements sends at an exact density (warm-up
    schedule), computed by the library's dgc_k_for_density."""
    num, den = _density_fraction(density)
    return dgc_k_for_density(n, num, den)


class Learner:
    """One learner's device state for a tensor layout: u, v, workspace and
    output buffers, as torch tensors on the current device."""

    def __init__(self, sizes: Sequence[int], k_max: Sequence[int],
                 momentum: float = 0.9, device="cuda", stream=None):
        import torch
        self.sizes = [int(s) for s in sizes]
        self.k_max = [int(x) for x in k_max]
        self.T = len(self.sizes)
        self.n = int(sum(self.sizes))
        dev = torch.device(device)
        self.u = torch.empty(max(self.n, 1), dtype=torch.float32, device=dev)
        self.v = torch.empty(max(self.n, 1), dtype=torch.float32, device=dev)
        ws = dgc_workspace_bytes(self.sizes, self.k_max)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.state = dgc_init_state(self.sizes, self.k_max, momentum, self.u,
                                    self.v, self.workspace, stream)
        K = max(int(sum(self.k_max)), 1)
        self.idx = torch.empty(K, dtype=torch.int32, device=dev)
        self.val = torch.empty(K, dtype=torch.float32, device=dev)
        self.norm = torch.empty(1, dtype=torch.float64, device=dev)
        self.scale = torch.empty(1, dtype=torch.float32, device=dev)
        self.cap = dgc_stream_capacity(self.state, self.T)
        C = max(int(self.cap[-1]), 1)
        self.runs = torch.empty(C, dtype=torch.int16, device=dev)
        self.vals = torch.empty(C, dtype=torch.float32, device=dev)
        self.entries = torch.empty(self.T, dtype=torch.int64, device=dev)
        self.count = torch.empty(self.T, dtype=torch.int64, device=dev)
        self.total = torch.empty(self.T, dtype=torch.int64, device=dev)

    def _check_grad(self, g):
        """The kernels read n floats from g: refuse a shorter or differently
        typed gradient here, before any launch."""
        import torch
        if g.dtype != torch.float32 or g.numel() < self.n:
            raise ValueError(f"gradient must be float32 with at least {self.n} elements "
                             f"(got {g.dtype}, {g.numel()})")

    def compress(self, g, k: Sequence[int], clip: float, stream=None):
        """One step; returns (idx, val) views holding sum(k) entries."""
        self._check_grad(g)
        K = int(sum(int(x) for x in k))
        dgc_compress(self.state, g, k, clip, self.idx, self.val, self.norm,
                     self.scale, stream)
        return self.idx[:K], self.val[:K]

    def compress_binlocal(self, g, bin_len: Sequence[int], cap: Sequence[int],
                          clip: float, stream=None):
        """One step with the bin-local selector.  Returns (idx, val, count,
        total): idx/val hold sum(cap) slots, tensor t's count[t] delivered
        entries first in its cap[t] slots; total[t] = salient entries."""
        self._check_grad(g)
        C = int(sum(int(x) for x in cap))
        dgc_compress_binlocal(self.state, g, bin_len, cap, clip, self.idx,
                              self.val, self.count, self.total, self.norm,
                              self.scale, stream)
        return self.idx[:C], self.val[:C], self.count, self.total

    def compress_sampled(self, g, k: Sequence[int], cap: Sequence[int], clip: float,
                         stream=None):
        """One step with the sampled threshold (about k[t] entries per
        tensor).  Returns (idx, val, count, total) as compress_binlocal."""
        self._check_grad(g)
        C = int(sum(int(x) for x in cap))
        dgc_compress_sampled(self.state, g, k, cap, clip, self.idx, self.val,
                             self.count, self.total, self.norm, self.scale, stream)
        return self.idx[:C], self.val[:C], self.count, self.total

    def compress_hier(self, g, k: Sequence[int], clip: float, stream=None):
        """One step with hierarchical thresholding (at most k[t] entries per
        tensor).  Returns (idx, val, count): idx/val hold sum(k) slots,
        tensor t's count[t] sent entries first in its k[t] slots."""
        self._check_grad(g)
        K = int(sum(int(x) for x in k))
        dgc_compress_hier(self.state, g, k, clip, self.idx, self.val, self.count,
                          self.norm, self.scale, stream)
        return self.idx[:K], self.val[:K], self.count

    def compress_shared(self, g, k: Sequence[int], shared_idx, clip: float, stream=None):
        """One step at another learner's index set (shared_idx: that
        learner's idx, sum(k) entries).  Returns the val view (sum(k))."""
        self._check_grad(g)
        K = int(sum(int(x) for x in k))
        dgc_compress_shared(self.state, g, k, shared_idx, clip, self.val, self.norm,
                            self.scale, stream)
        return self.val[:K]

    def encode_counts(self, cap: Sequence[int], stream=None):
        """Encode what compress_binlocal delivered (counts on the device)."""
        dgc_encode_counts(self.state, cap, self.count, self.idx, self.val,
                          self.runs, self.vals, self.entries, stream)
        return self.runs, self.vals, self.entries

    def encode(self, k: Sequence[int], stream=None):
        dgc_encode(self.state, k, self.idx, self.val, self.runs, self.vals,
                   self.entries, stream)
        return self.runs, self.vals, self.entries

    def set_option(self, option: int, value: int):
        dgc_set_option(self.state, option, value)

    def set_fused_event(self, event):
        dgc_set_fused_event(self.state, event)

    def status(self) -> int:
        return dgc_get_status(self.state)

    def path_counts(self) -> Tuple[int, int]:
        return dgc_get_path_counts(self.state)

    def select_info(self) -> np.ndarray:
        return dgc_get_select_info(self.state, self.T)

    def kernel_time(self, timer: int) -> Tuple[float, int]:
        return dgc_get_kernel_time(self.state, timer)

    def close(self):
        if self.state is not None:
            dgc_destroy_state(self.state)
            self.state = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_accumulate(layout_learner: Learner, streams: List[Tuple], dense,
                      stream=None):
    """dense += the decoded streams [(runs, vals, entries), ...] in order."""
    dgc_decode_accumulate(layout_learner.state, [s[0] for s in streams],
                          [s[1] for s in streams], [s[2] for s in streams],
                          dense, stream)


def decode_sum(layout_learner: Learner, streams: List[Tuple], dense, stream=None):
    """dense = the decoded streams [(runs, vals, entries), ...] summed in order
    from +0.0 (every element of dense is written)."""
    dgc_decode_sum(layout_learner.state, [s[0] for s in streams],
                   [s[1] for s in streams], [s[2] for s in streams], dense, stream)


def shared_sum(layout_learner: Learner, vals: Sequence, k: Sequence[int], shared_idx,
               out_sum, dense=None, stream=None):
    """out_sum = the learners' value vectors summed in learner order from +0.0;
    dense (optional) = out_sum scattered at shared_idx, +0.0 elsewhere."""
    dgc_shared_sum(layout_learner.state, vals, k, shared_idx, out_sum, dense, stream)
