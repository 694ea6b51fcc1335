"""MI355X-native top-k Mixture-of-Experts layer forward.

The layer runs in hand-written HIP kernels for gfx950 behind a C ABI
(``include/moe.h``); ``expert_ffn_layer_router_amd.binding`` is the thin ctypes
layer over it that takes torch device tensors. Importing this package loads
nothing; the shared library is loaded on the first call into the binding, and
that call raises if the library has not been built.
"""

__all__ = ["binding", "accounting"]
