"""libfa: exact FlashAttention forward pass for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI shared library ``libfa.so`` (hand-written HIP
kernels, declared in ``include/fa.h``); ``exact_attention_13_amd.binding`` is a
thin ctypes binding over it.  PyTorch is used only to own device memory and
streams.  Importing this package does not load the library; the first call
of ``fwd`` does, and fails loudly if it is missing.
"""
__all__ = ["fwd", "fa_fwd", "version"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
