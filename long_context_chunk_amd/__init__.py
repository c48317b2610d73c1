"""HiLS-Attention forward pass on AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``libhils.so`` (include/hils.h) built from the
HIP sources in ``csrc/``; ``hils`` is its Python binding.
"""
