"""libqar: dynamic block-wise int8 quantized reduction on MI355X (gfx950).

The compute lives in the HIP shared library ``libqar.so`` built from
``csrc/``; ``qar`` is its ctypes binding.  Importing the package loads
nothing: the library is opened on first use and a missing library raises.
"""
