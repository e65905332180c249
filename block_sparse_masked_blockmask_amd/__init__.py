"""Block-sparse masked attention forward and backward for MI355X (gfx950).

The computation lives in libflexattn.so (HIP kernels behind the C ABI of
include/flexattn.h); `flexattn` is its ctypes binding with the same entry-point names.
"""
from .flexattn import (  # noqa: F401
    FA_BF16, FA_F32, FA_FP8_E4M3, FA_I8,
    FA_MASK_CAUSAL, FA_MASK_DOC, FA_MASK_NONE, FA_MASK_PREFIX_LM, FA_MASK_WINDOW,
    FA_SCORE_ALIBI, FA_SCORE_NONE, FA_SCORE_SOFTCAP,
    FA_OK, FA_ERR_DEVICE, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED,
    BlockMask, BlockMaskTransposed, FlexAttnError, LIB_PATH, block_mask_all_partial,
    flexattn_block_mask_build, flexattn_block_mask_build_host, flexattn_block_mask_build_noalloc,
    flexattn_block_mask_bytes, flexattn_block_mask_noalloc_max_bytes,
    flexattn_block_mask_count_bytes, flexattn_fwd_workspace_bytes,
    flexattn_block_mask_index_bytes, flexattn_block_mask_transpose, flexattn_bwd, flexattn_bwd_workspace_bytes,
    flexattn_block_mask_workspace_bytes, flexattn_fwd, flexattn_fwd_splitkv, flexattn_fwd_splitkv_workspace_bytes,
    flexattn_fwd_quant, flexattn_last_error, flexattn_quantize_qkv, flexattn_quantize_qkv_ex,
    flexattn_quantize_qkv_ex_workspace_bytes,
    flexattn_version,
    lib, tensor_desc,
)
