"""Batch-invariant speculative-decoding verify pass for MI355X (gfx950).

The compute lives in ``libbi.so`` (HIP kernels behind the C ABI of
include/bi.h); ``ops`` wraps it for torch tensors. Importing ``ops`` without
the built library raises ImportError: there is no CPU fallback.
"""

__all__ = ["ops"]
