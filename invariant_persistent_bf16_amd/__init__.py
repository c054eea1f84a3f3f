"""Batch-invariant dense contractions for AMD Instinct MI355X (gfx950).

The product is the C-ABI library libbi.so (include/bi.h); ``bi`` is its thin
ctypes binding.  Importing this package loads nothing; ``from
invariant_persistent_bf16_amd import bi`` loads the binding, whose first call
loads the library (and raises if it has not been built).
"""
