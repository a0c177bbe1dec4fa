"""MI355X (gfx950) Hadamard-quantized linear-layer matmul (HQ-MM / HALO-2).

The computation lives in libhq.so (hand-written HIP kernels behind the C ABI of
include/hq.h); ``binding`` exposes the same entry-point names through ctypes, ``tensors``
allocates device memory with torch, and ``workloads`` draws the seeded synthetic inputs.
"""
from . import binding  # noqa: F401

__all__ = ["binding", "build", "tensors", "workloads"]
