"""QSA (Qwen Sparse Attention) decode path for AMD MI355X (gfx950).

libqsa.so holds the HIP kernels behind a C ABI (include/qsa.h); `qsa` is its Python
binding and `inputs` the seeded synthetic workload generator. Importing the package
loads nothing; `qsa` loads the library on first use.
"""
__all__ = ["qsa", "inputs"]
