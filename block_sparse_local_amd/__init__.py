"""MI355X-native banded block-sparse attention forward.

The compute path lives in ``libbsl.so`` (hand-written gfx950 HIP kernels behind
a C ABI, declared in ``include/bsl.h``); ``block_sparse_local_amd.bsl`` is a
thin ctypes binding with the same names.  Nothing here falls back to another
implementation: calling the binding without the built library raises.
"""
__all__ = ["bsl", "inputs", "workload"]
