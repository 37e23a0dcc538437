"""Token Sparse Attention prefill on MI355X (gfx950): HIP kernels behind a C ABI.

``tsa`` holds the binding (same names as include/tsa.h); ``inputs`` the seeded
synthetic workloads; ``build`` compiles libtsa.so in-tree.
"""
__version__ = "0.1.0"
