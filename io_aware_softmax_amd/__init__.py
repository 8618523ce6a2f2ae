"""Exact attention forward for AMD MI355X (gfx950).

The computation lives in ``libattn.so`` (HIP kernels behind the C ABI of
``include/attn.h``); ``binding`` marshals torch tensors into it.  Submodules:

* ``binding``: ``attn_fwd``, ``attn_decode_fwd``, ``attn_decode_auto_splits``,
  ``attn_strerror`` (the C ABI's names), ``AttnError``;
* ``inputs``: seeded synthetic workloads (no attention arithmetic);
* ``build``: compiles the library in-tree with hipcc for gfx950.

The binding is imported on first attribute access so that ``inputs`` can be
used without loading torch's GPU runtime.
"""

_BINDING_NAMES = ("attn_fwd", "attn_decode_fwd", "attn_decode_auto_splits", "attn_strerror",
                  "AttnError", "AttnLibraryMissing", "load", "raw_attn_fwd", "raw_attn_decode_fwd")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
