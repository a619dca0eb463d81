"""MI355X-native hybrid compressed attention (CSA / HCA).

The compute lives in a C-ABI shared library of hand-written HIP kernels for gfx950
(``libcsa.so``, built from ``csrc/``); ``ops`` is a thin ctypes binding with the same
entry-point names.  Importing the package loads nothing; ``ops`` loads the library on
first use and raises if it is missing.
"""

__all__ = ["configs", "synth", "ops"]
