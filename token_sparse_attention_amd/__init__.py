"""Token Sparse Attention prefill layer for MI355X (gfx950): HIP kernels behind a C ABI (libtsa.so)
and a thin ctypes binding.  Importing the package loads nothing; the library is opened on first use
and a missing library is an error, never a fallback."""

from .configs import WORKLOADS, Workload  # noqa: F401
