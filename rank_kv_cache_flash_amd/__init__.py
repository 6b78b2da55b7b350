"""WSVD per-head low-rank flash decoding on MI355X (gfx950).

The compute lives in ``libwsvd.so`` (hand-written HIP, C ABI declared in
``include/wsvd.h``); ``rank_kv_cache_flash_amd.wsvd`` marshals torch
tensors into it.  Importing this package loads nothing; the library is
loaded on first use and a missing library is an error, never a fallback.
"""
__all__ = ["wsvd", "inputs", "configs"]
