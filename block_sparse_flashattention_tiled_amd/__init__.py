"""Block-sparse FlashAttention prefill (BSFA form) for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libbsfa.so``, built from ``csrc/``); :mod:`.binding` marshals torch device
tensors into its entry points.  Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""

from . import accounting, workloads  # noqa: F401

__all__ = ["accounting", "workloads"]
