"""Frame-aligned windowed sparse attention for AMD Instinct MI355X (gfx950).

The compute lives in libfsa.so (HIP kernels behind the C ABI of
include/fsa.h); ``fsa`` is its ctypes binding and ``inputs`` the seeded
synthetic workload generator.
"""
