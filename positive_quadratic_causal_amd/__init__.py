"""MI355X-native OAL (Outlier-Aware Attention Linearization) causal attention.

The compute path lives in ``liboal.so`` (hand-written HIP kernels for gfx950
behind a C ABI declared in ``include/oal.h``); ``positive_quadratic_causal_amd.oal``
is the thin ctypes binding.  Importing this package itself loads nothing, so the
seeded input generator (``synth``) can be used on hosts without a GPU.
"""
__version__ = "0.1.0"
