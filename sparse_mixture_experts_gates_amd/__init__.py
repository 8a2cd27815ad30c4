"""MI355X-native sparse mixture-of-experts feed-forward layer (forward pass).

The compute lives in ``libmoe_mi355x.so`` (hand-written HIP kernels for gfx950
behind a C ABI declared in ``include/moe.h``).  ``binding`` marshals torch
tensors into that ABI; ``workloads`` draws seeded synthetic inputs.  Importing
this package does not load the library; the first call into ``binding`` does,
and raises if it has not been built.
"""

__all__ = ["binding", "workloads"]
