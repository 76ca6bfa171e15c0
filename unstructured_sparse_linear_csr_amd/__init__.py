"""MI355X-native unstructured-sparse CSR kernels: SpMM and SDDMM.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, declared in ``include/sp_csr.h``).  ``binding`` is a thin
ctypes layer over it that marshals torch tensors (device memory and streams
only).  ``inputs`` holds the seeded synthetic workloads.

Importing the package loads nothing; ``binding`` loads the library on first
use and raises if it is missing.
"""

__all__ = ["binding", "inputs"]
