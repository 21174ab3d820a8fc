"""SparsePR per-call sparse attention operator for AMD MI355X (gfx950).

The compute path is the HIP library ``libsparsepr.so`` (C-ABI declared in
``include/sparsepr.h``); ``binding`` marshals torch tensors into it. Importing
this package does not load the library; ``binding.load()`` does, and fails
loudly when it is missing.
"""
__all__ = ["configs", "inputs", "binding"]
