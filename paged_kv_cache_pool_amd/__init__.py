"""Paged-attention step for AMD Instinct MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``).  ``paged_kv_cache_pool_amd.binding`` is a thin
ctypes layer over that library; ``workloads`` draws seeded synthetic inputs.
"""
