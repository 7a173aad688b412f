"""Hybrid block-sparse + ReLU-linear attention (SALAD-style) for AMD MI355X.

The operator lives in the HIP library ``libsalad.so`` (C interface in
include/salad.h); ``block_sparse_linear_st_amd.salad`` is its ctypes binding
and ``block_sparse_linear_st_amd.layer`` a small convenience wrapper that owns
the device buffers of one layer.
"""

from . import salad  # noqa: F401
