"""Exact scaled dot-product attention (forward + backward) for MI355X / gfx950.

The compute path is libexattn.so (hand-written HIP kernels behind the C ABI in
include/exattn.h); this package only marshals PyTorch device tensors into it.
"""

from ._binding import (  # noqa: F401
    EXATTN_BF16,
    EXATTN_F32,
    EXATTN_FP8_ROWS,
    EXATTN_FP8_V_TRANSPOSED,
    EXATTN_NOALLOC_SCRATCH_BYTES,
    AttnPattern,
    ExattnError,
    LIB_PATH,
    attn_bwd,
    attn_bwd_dkdv,
    attn_bwd_dkdv_gqa,
    attn_bwd_dq,
    attn_bwd_dq_gqa,
    attn_bwd_gqa,
    attn_bwd_noalloc,
    attn_bwd_pattern,
    attn_bwd_rowdot,
    attn_bwd_workspace_bytes,
    attn_fwd,
    attn_fp8_bytes,
    attn_fwd_fp8,
    attn_fwd_gqa,
    attn_fwd_pattern,
    attn_pattern_workspace_bytes,
    attn_quant_fp8,
    exattn_status_string,
    load_library,
)
