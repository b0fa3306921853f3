"""MI355X-native Geometric Context Attention (GCA) step with a paged KV cache.

The compute path lives in libgca.so (HIP kernels for gfx950 behind the C ABI
declared in include/gca.h); ``_lib`` is its ctypes binding and ``synth`` the
seeded input generator shared by tests and benchmark.
"""
