"""MI355X-native split-KV decode attention (FlashDecoding) for gfx950.

The compute path is the HIP library ``libfd.so`` (C ABI, see include/fd.h);
``decode_attention_03_amd.fd`` is its thin Python binding.  Importing the package
loads nothing: the library is opened on the first call of the binding, and a
missing library is an error there, never a silent fallback.
"""
__all__ = ["fd", "workloads"]
