"""libgqa: fused causal grouped-query attention for AMD MI355X (gfx950).

The hot path lives in the C-ABI shared library ``libgqa.so`` (HIP kernels,
``include/gqa.h``); this package is its ctypes binding.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    GQA_BF16,
    GQA_F16,
    GQA_F32,
    GqaAttention,
    GqaError,
    abi_version,
    gqa_attention,
    gqa_attn_bwd,
    gqa_attn_bwd_dkdv,
    gqa_attn_bwd_dq,
    gqa_attn_bwd_grads,
    gqa_attn_bwd_preprocess,
    gqa_attn_bwd_workspace_bytes,
    gqa_attn_decode,
    gqa_attn_decode_workspace_bytes,
    gqa_attn_fwd,
    gqa_decode_problem,
    gqa_problem,
    gqa_visible_pairs,
    library,
    make_decode_problem,
    make_problem,
    status_str,
)
