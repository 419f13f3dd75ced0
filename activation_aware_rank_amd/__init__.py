"""Activation-aware low-rank compression on MI355X (gfx950).

The compute path lives in the HIP library ``liblrc.so`` built from ``csrc/``; the
``lrc`` module is its thin ctypes binding.  Importing this package loads nothing:
``from activation_aware_rank_amd import lrc`` loads the library and raises if it
has not been built.
"""
__all__ = ["lrc", "inputs"]
