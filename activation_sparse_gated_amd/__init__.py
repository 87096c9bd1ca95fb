"""Gate-first sparse FFN forward pass for AMD MI355X (gfx950).

The compute path is the HIP library ``libsffn.so`` (C ABI declared in
``include/sffn.h``); ``activation_sparse_gated_amd.sffn`` is its thin ctypes
binding. Importing this package loads nothing: the library is opened on the
first call into the binding, which fails loudly if it has not been built.
"""
__all__ = ["sffn", "inputs"]
