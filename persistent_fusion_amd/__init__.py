"""Persistent small-op runtime for AMD Instinct MI355X (gfx950).

The runtime itself is native: ``csrc/`` holds the HIP kernels and the host
runtime behind the C ABI declared in ``include/gpuos.h``; :mod:`.gpuos` is a
thin ctypes binding over that library.  :mod:`.workloads` draws seeded
synthetic op queues and :mod:`.traffic` is the algorithmic byte model used for
effective bandwidth.
"""

__all__ = ["gpuos", "workloads", "traffic"]
