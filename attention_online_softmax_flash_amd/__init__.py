"""Fused inference attention for AMD Instinct MI355X (gfx950).

The compute path is libfia.so (HIP kernels + host planner, C ABI in
include/fia.h); ``fia`` is its ctypes binding and ``torch_io`` turns the
seeded workloads of ``workloads`` into device tensors and plans.
"""
from . import workloads  # noqa: F401  (numpy only; no GPU needed)

__all__ = ["workloads", "fia", "torch_io"]
