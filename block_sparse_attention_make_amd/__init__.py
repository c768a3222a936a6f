"""MI355X-native splash-attention forward: block-sparse, mask-aware flash
attention whose loop structure is read from a compiled MaskInfo.

    from block_sparse_attention_make_amd import make_mask_info, splash_fwd
    mi = make_mask_info("causal", 8192, 8192)
    out, lse = splash_fwd(q, k, v, mi)          # q, k, v: GPU bf16 [B, H, S, D]

The native library (libsplash.so: HIP kernels for gfx950, the host mask
compiler and the C ABI of include/splash.h) is loaded on first use and must
have been built with `python -m block_sparse_attention_make_amd.build`.
"""
from .splash import (MaskInfo, SplashError, load_library, lse_merge, make_mask_info,  # noqa: F401
                     splash_attention, splash_bwd, splash_decode, splash_decode_static, splash_fwd,
                     splash_fwd_kv_sharded)
