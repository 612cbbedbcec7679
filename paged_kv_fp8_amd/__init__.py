"""Paged-KV e4m3 decode attention for AMD MI355X (gfx950).

The compute lives in ``libpkvfp8.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/pkv_fp8.h``). ``paged_kv_fp8_amd.native`` is the
thin ctypes binding with the same entry-point names; importing it loads the
library and fails loudly if it has not been built. ``workloads`` generates
seeded synthetic batches in the tensor contract.
"""

__all__ = ["native", "workloads"]
