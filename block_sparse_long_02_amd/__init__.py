"""MI355X-native QSA (Qwen Sparse Attention) hot path.

The compute lives in ``libqsa.so`` (hand-written HIP kernels for gfx950 behind
a C ABI declared in ``include/qsa.h``); ``block_sparse_long_02_amd.qsa`` is a
thin ctypes binding with the same entry-point names.  ``workloads`` builds
seeded synthetic inputs.
"""
__all__ = ["qsa", "workloads"]
