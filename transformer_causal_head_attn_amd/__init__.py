"""libattn: multi-head scaled-dot-product self-attention, forward and
backward, on AMD Instinct MI355X (gfx950) with hand-written HIP kernels.

The compute lives in ``libattn.so`` (C ABI: ``include/libattn.h``); this
package only builds it and marshals torch tensors into its calls.  Importing
the package does not load the library; the first call does, and fails loudly
if it cannot.
"""
from ._binding import (  # noqa: F401
    ATTN_EHIP, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_OK, EXPORTS, LIB_PATH, AttnError,
    attn_backward, attn_backward_bf16, attn_backward_dkdv, attn_backward_dkdv_bf16,
    attn_backward_noalloc, attn_backward_prepare, attn_backward_dkdvdq,
    attn_forward_splitkv_chunk, attn_forward_splitkv_bytes,
    attn_forward_splitkv_bf16, attn_forward_splitkv_f16, forward_splitkv,
    attn_backward_splitkv_bytes, attn_backward_splitkv_bf16, attn_backward_splitkv_f16,
    backward_splitkv,
    attn_qkv_projection, attn_qkv_projection_bf16, attn_out_projection, attn_out_projection_bf16,
    qkv_projection, out_projection,
    attn_backward_dq, attn_backward_dq_bf16, attn_backward_materialized,
    attn_backward_ds_bytes, attn_backward_dkdv_ds, attn_backward_dq_ds,
    attn_backward_preprocess, attn_backward_preprocess_bf16, attn_decode, attn_decode_bf16, attn_decode_f16,
    attn_backward_dkdv_f16, attn_backward_dq_f16, attn_backward_f16,
    attn_backward_preprocess_f16, attn_forward_f16, attn_forward_fp8, forward_fp8,
    attn_forward, attn_forward_bf16, attn_forward_materialized, attn_last_error, attn_merge,
    attn_merge_bf16, attn_merge_f16, attn_release, attn_set_stream, backward, backward_materialized, decode,
    forward, forward_materialized, load, merge,
    layernorm, layernorm_backward, layernorm_backward_bf16, layernorm_forward,
    layernorm_forward_bf16, layernorm_grad, layernorm_forward_f16, layernorm_backward_f16,
)
