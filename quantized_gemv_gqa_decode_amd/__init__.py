"""MI355X-native batch-1 decode hot path: quantized GEMV + GQA decode attention.

The compute lives in ``libk2.so`` (hand-written HIP for gfx950, C ABI in
``include/k2.h``); ``k2`` is its ctypes binding and ``model`` keeps a whole
decoder's device buffers.
"""
from . import k2  # noqa: F401

__all__ = ["k2"]
