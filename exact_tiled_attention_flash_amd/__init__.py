"""MI355X-native exact tiled attention (FlashAttention forward and backward).

The compute lives in hand-written HIP kernels for gfx950 behind the C ABI
declared in include/fa.h (libfa.so); this package is a thin ctypes binding
over it with the same entry-point names. Importing it loads libfa.so and
fails loudly if the library has not been built.
"""
from ._lib import (  # noqa: F401
    FA_BF16,
    FA_F32,
    FaError,
    LIB_PATH,
    fa_abi_version,
    fa_bwd,
    fa_bwd_noalloc,
    fa_bwd_noalloc_max_bytes,
    fa_bwd_workspace_bytes,
    fa_decode_workspace_bytes,
    fa_fwd,
    fa_fwd_decode,
    fa_fwd_fp8qk,
    fa_fwd_gqa,
    fa_fwd_varlen,
    fa_quantize_mxfp8,
    fa_status_string,
    load_library,
)

load_library()
