"""libssd: the Mamba-2 SSD layer (forward, backward, recurrent step) on MI355X (gfx950),
behind a C ABI.

The compute path is the HIP library `libssd.so` in this package directory (built by
`build.py`); `binding` is a thin ctypes layer over it.  Importing the package does not
load the library; the first call through `binding` does, and fails loudly if it is
missing.
"""
from .workloads import WORKLOADS, STRESS, Workload, generate  # noqa: F401

__all__ = ["WORKLOADS", "STRESS", "Workload", "generate"]
