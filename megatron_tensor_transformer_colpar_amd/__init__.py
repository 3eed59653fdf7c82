"""MI355X-native per-rank share of a Megatron tensor-parallel MLP block.

The compute path is the HIP library ``libtpcolpar.so`` (sources in ``csrc/``,
C header ``include/tp_colpar.h``); ``tp`` is its thin ctypes binding and raises
if the library has not been built.  ``inputs`` draws the seeded synthetic
tensors.  Importing this package loads nothing native.
"""
__all__ = ["inputs", "tp"]
