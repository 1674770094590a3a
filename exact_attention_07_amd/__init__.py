"""MI355X-native fused exact attention: forward and backward passes.

The compute path is the C-ABI library libfa.so (hand-written HIP kernels for
gfx950, declared in include/fa.h).  `exact_attention_07_amd.api` is a thin
ctypes binding with the same entry-point names; `exact_attention_07_amd.gen`
is the seeded synthetic input generator.  Importing this package loads
nothing; the binding loads the library on first use and raises if it is
missing.
"""
__all__ = ["api", "gen"]
