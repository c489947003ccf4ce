"""MI355X (gfx950) tiled online-softmax attention.

The compute lives in the HIP library ``libfa.so`` (built from ``csrc/``);
``fa`` is its thin ctypes binding.  Importing this package does not load the
library: the first call does, and fails loudly if it is missing.
"""
