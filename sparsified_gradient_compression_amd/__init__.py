"""Per-learner sparsifying gradient compressor (Deep Gradient Compression
family) for MI355X: a C-ABI library of hand-written HIP kernels for gfx950
and a thin ctypes binding with the same entry-point names."""
