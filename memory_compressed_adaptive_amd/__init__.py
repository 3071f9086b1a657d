"""MicroAdam optimizer step on AMD Instinct MI355X (gfx950).

The step of the page "MicroAdam (Sparse-Gradient Adaptive Optimization with
Quantized Error Feedback)" runs in the HIP kernels of libmicroadam.so (C ABI:
include/microadam.h); this package holds the ctypes binding (`MicroAdam`), the
build script and the synthetic workloads used to benchmark it.
"""
from ._lib import MicroAdamError, lib  # noqa: F401
from .optimizer import MicroAdam  # noqa: F401
