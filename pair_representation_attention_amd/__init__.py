"""MI355X (gfx950) pair-biased attention: triangle attention around the
starting and ending node, and MSA row attention with a pair bias.

The compute lives in the HIP shared library ``libpairattn.so`` (C ABI,
declared in ``include/pairattn.h``).  ``pair_representation_attention_amd.lib``
is a thin ctypes binding over it with the same entry-point names; it loads
the library on first use and raises if it is missing.
"""
__all__ = ["inputs", "lib"]
