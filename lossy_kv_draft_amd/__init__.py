"""Python binding of the VeriCache hot-path library (libvc.so, HIP for gfx950).

Argument marshalling only: every function forwards to the C entry point of the same
name in include/vc.h.  Tensors are torch tensors (device memory on the current HIP
device, pinned host memory for staging sources); streams are torch.cuda.Stream
objects or None for the current stream.  The library is loaded from this package
directory; importing fails loudly when it has not been built.
"""
from ._lib import (  # noqa: F401
    VcError, lib, LIB_PATH, VC_F32, VC_BF16, VC_QUANT_KIVI, VC_DROP_TOPK, EXPORTS,
    Ckv, vc_ckv_sizes, vc_workspace_size, CKV_ARRAYS, VC_CKV_DECODE_F32, VC_OP_COMPRESS, VC_OP_DECODE,
    VC_OP_VERIFY, VC_OP_LOGITS, vc_compress, vc_compress_workspace_bytes, vc_drop_keep_count, vc_drop_scores,
    vc_drop_scores_workspace_bytes, vc_drop_select, vc_gather_rows, vc_decode_attn_compressed,
    vc_decode_workspace_bytes, vc_decode_attn_compressed_noalloc, VC_DECODE_NOALLOC_SCRATCH_BYTES,
    vc_verify_attn_full, vc_verify_workspace_bytes, vc_verify_split_tokens,
    vc_head_mean, vc_logits_argmax, vc_logits_workspace_bytes, vc_accept, vc_stage_full_kv, vc_hadamard_rows,
    vc_stage_full_kv_d2h, vc_last_error, workspace, FileStager, VC_ERR_IO,
    vc_split_planes, vc_join_planes, split_residuals,
    vc_gemm_bf16_swiglu, swiglu_interleave, vc_gemm_bf16_rope, rope_interleave,
    vc_gemm_bf16, vc_gemm_bf16_wide, vc_rmsnorm, vc_rope_qkv, vc_swiglu, vc_embed, vc_heads_to_rows, vc_argmax_rows, vc_copy_kv_rows,
)
