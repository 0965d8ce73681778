"""WISE working-set attention for MI355X (gfx950).

The compute path lives in the HIP library ``libwise.so`` (C ABI declared in
``include/wise.h``); :mod:`block_sparse_attention_wise_amd.wise` is its thin
Python binding and :mod:`block_sparse_attention_wise_amd.synthetic` the seeded
input generator.  Importing the package itself loads nothing.
"""
__all__ = ["wise", "synthetic"]
