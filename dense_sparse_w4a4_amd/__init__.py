"""MI355X-native fused W4A4 + block-sparse INT4 residual linear layer.

The compute lives in ``libmosaicq.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/mosaicq.h``).  ``dense_sparse_w4a4_amd.ops`` is a thin
ctypes binding over it; torch tensors only provide device memory and streams.
Importing this package does not load the library; the first call does, and
raises if it has not been built.
"""
__all__ = ["ops", "synthetic"]
