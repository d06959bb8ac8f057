"""Brute-force NumPy / Python versions of each step, for tiny inputs.

TEST INFRASTRUCTURE ONLY.  These exist to pin the C++ oracle with methods
that share nothing with it: top-k by a full sort instead of a selection
algorithm, the encoder as a walk over every index of the tensor instead of a
walk over the selected list, decoding with ``np.add.at``.  Each follows the
DGC review page ("Deep Gradient Compression: Reducing the Communication
Bandwidth for Distributed Training", section "Proposed method").
"""

import numpy as np


def magnitude_keys(v):
    """|v| as the IEEE bit pattern with the sign bit cleared (uint32)."""
    return v.astype(np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)


def topk_fullsort(v, k):
    """Local indices (ascending) of the k entries first under
    (|v| descending, index ascending), by sorting every entry."""
    keys = magnitude_keys(v).astype(np.int64)
    order = np.lexsort((np.arange(v.size), -keys))
    return np.sort(order[:k]).astype(np.uint32)


def encode_walk(n, idx, val):
    """Encode by walking every position 0..n-1 and counting zeros.

    A zero run is closed by a selected entry; a run that reaches 65535
    zeros while the next position is also unselected emits a filler entry
    (65535, 0.0) that consumes that next position as well.
    """
    sel = {int(i): np.float32(x) for i, x in zip(idx, val)}
    last = max(sel) if sel else -1
    runs, vals = [], []
    zeros = 0
    for pos in range(last + 1):
        if pos in sel:
            runs.append(zeros)
            vals.append(sel[pos])
            zeros = 0
        elif zeros == 65535:
            runs.append(65535)
            vals.append(np.float32(0.0))
            zeros = 0
        else:
            zeros += 1
    return np.array(runs, np.uint16), np.array(vals, np.float32)


def decode_positions(runs):
    """Positions of the entries of one stream: cumulative (run + 1) - 1."""
    return np.cumsum(runs.astype(np.int64) + 1) - 1


def decode_accumulate_addat(streams, n):
    """Sum of several learners' streams into a dense float32 vector, learner
    by learner in order, with ``np.add.at``."""
    dense = np.zeros(n, np.float32)
    for runs, vals in streams:
        pos = decode_positions(runs)
        assert pos.size == 0 or pos[-1] < n
        np.add.at(dense, pos, vals.astype(np.float32))
    return dense
