"""MI355X-native band + global sparse self-attention (forward).

The compute path is the C-ABI library ``liblfattn.so`` (hand-written HIP
kernels for gfx950, declared in ``include/lfattn.h``); ``lfattn`` is its thin
ctypes binding.  ``workloads`` makes the seeded synthetic inputs.  Nothing is
loaded at import time: the binding opens the library on first use and raises
if it is missing.
"""

__all__ = ["lfattn", "workloads"]
