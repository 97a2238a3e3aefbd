"""CPU oracle (float64 NumPy) for paged decode and prefill attention, the cache
write and the page copy.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its Python binding.
It shares no code with the HIP path.  Every function is pinned by CPU tests
(brute force, closed forms, invariants, a library routine, the pages'
page-table figure); no function is "parity unpinned".
"""
from .paged_attention import (copy_blocks, decode, gather_pages, prefill, reshape_and_cache, rope,
                              widen)

__all__ = ["copy_blocks", "decode", "gather_pages", "prefill", "reshape_and_cache", "rope", "widen"]
