"""CSA2 sparse-attention hot path for AMD MI355X (gfx950).

The compute lives in ``libcsa2.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/csa2.h``).  ``binding`` exposes the entry points under
the same names; ``runner`` allocates a workload's device buffers with torch.
Importing ``binding`` fails if the library has not been built.
"""

__all__ = ["binding", "runner"]
