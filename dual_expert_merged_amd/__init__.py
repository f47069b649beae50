"""MI355X-native DM0-style dual-expert merged-attention path.

The compute lives in a HIP library (``libdm.so``, C ABI in ``include/dm.h``); ``binding``
marshals PyTorch device tensors into its calls.  Importing the package loads nothing; the
library is loaded on first use and its absence is an error, never a fallback.
"""
__all__ = ["configs", "inputs", "binding"]
