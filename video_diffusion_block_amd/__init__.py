"""MI355X (gfx950) block-sparse attention for video-DiT latent tokens.

The compute lives in ``libbsa.so`` (hand-written HIP, C ABI in include/bsa.h);
``ops`` wraps each entry point for torch device tensors. Importing the package
does not load the library; the first call does, and raises if it is missing.
"""
from . import ops  # noqa: F401
from .ops import (  # noqa: F401
    BSALayout,
    attn_bwd,
    attn_bwd_raster,
    attn_fwd,
    attn_fwd_gather,
    gather_supported,
    attn_fwd_raster,
    permute,
    permute_norm_rope,
    permute_pool,
    pool_select,
    select,
    select_causal,
    unpermute,
    xattn_bwd,
    xattn_fwd,
    zone_score,
)
from .schedule import ReusedSelection, refresh_steps  # noqa: F401
