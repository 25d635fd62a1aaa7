"""MI355X-native ring-decomposed all-gather + GEMM and GEMM + reduce-scatter.

The compute path is the HIP library libringag.so (csrc/, C ABI in include/ringag.h); this package
holds its thin ctypes binding (`binding`), the in-tree build step (`build`) and the seeded input
generators (`workloads`).  Importing the package loads nothing; the first call into the binding
loads the library and raises if it has not been built.
"""

__all__ = ["binding", "workloads", "build"]
