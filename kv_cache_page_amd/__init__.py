"""LOCKS decode hot path on AMD Instinct MI355X (gfx950).

Page-local spectral key summaries score and select paged-KV pages, then a
sparse decode attention reads only the selected pages. All computation runs
in the HIP library behind include/locks.h; `kv_cache_page_amd.locks` is its
ctypes binding.
"""
__all__ = ["locks"]
