"""DMS (Dynamic Memory Sparsification) inference hot path for AMD MI355X (gfx950).

The compute lives in libdms.so (HIP kernels behind the C ABI of include/dms.h);
``learned_kv_cache_amd.dms`` is its ctypes binding and
``learned_kv_cache_amd.synth`` the seeded synthetic input generator.  Importing
the package loads nothing; the library is loaded on first use.
"""
__all__ = ["dms", "synth", "build"]
