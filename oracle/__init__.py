"""CPU oracle for the per-learner DGC compressor.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library (``sparsified_gradient_compression_amd``) and imports
nothing from it.

Two independent implementations live here:

* ``dgc_oracle.cpp`` (ctypes, module ``oracle.c_oracle``): the oracle the GPU
  results are compared with, fast enough for full-size workloads.
* ``oracle.bruteforce``: pure NumPy / Python brute force for tiny inputs
  (full sort for top-k, Python loops for the encoder), used to pin the C
  oracle.
"""

from .c_oracle import (  # noqa: F401
    build,
    lib_path,
    load,
    clip_scale,
    momentum,
    select_mask,
    encode,
    decode_accumulate,
    k_for_density,
    step,
    num_threads,
    set_num_threads,
    binlocal_select_mask,
    binlocal_step,
    fmix32,
    sampled_select_mask,
    sampled_step,
    hier_select_mask,
    hier_step,
    shared_gather_mask,
    shared_step,
    shared_sum,
)
