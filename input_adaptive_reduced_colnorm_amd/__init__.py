"""Reduced Matrix Multiplication (RMM) for AMD Instinct MI355X (gfx950).

The compute path lives in librmm.so (hand-written HIP, C ABI in
include/rmm.h); this package holds its build script and a thin binding.
"""

from .rmm import RMMError, k, lib, matmul, pv, qk, select, status_str  # noqa: F401
