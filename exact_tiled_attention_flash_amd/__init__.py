"""MI355X-native exact tiled attention (FlashAttention forward and backward).

The compute lives in hand-written HIP kernels for gfx950 behind the C ABI
declared in include/fa.h (libfa.so); this package is a thin binding over it.
"""
