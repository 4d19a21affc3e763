"""Exact tiled attention forward for MI355X (gfx950): a C-ABI HIP library (libfa.so,
include/fa.h) and its thin Python binding."""
from .fa import (FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_FP8_E4M3, FA_ERR_INVALID_ARG, FA_ERR_LAUNCH,
                 FA_ERR_UNSUPPORTED, FA_OK, FP8_BLOCK_ROWS, SPARSE_BLOCK, FaError, bwd, fa_bwd,
                 fa_bwd_workspace_bytes, fa_fwd, fa_fwd_block_sparse, fa_fwd_fp8_block, fa_fwd_local, fa_fwd_splitkv, fa_fwd_splitkv_workspace_bytes, fwd_splitkv,
                 fa_fwd_splitkv_static, fwd_splitkv_static, FA_ERR_SCRATCH, SPLITKV_STATIC_SCRATCH_BYTES,
                 fa_fwd_query, fa_quantize_e4m3_block, fwd, fwd_block_sparse, fwd_fp8_block, quantize_e4m3_block,
                 status_string, version)

__all__ = ["fwd", "fwd_block_sparse", "fa_fwd_block_sparse", "SPARSE_BLOCK", "bwd", "fwd_splitkv", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes", "fa_fwd_splitkv_static", "fwd_splitkv_static", "FA_ERR_SCRATCH", "SPLITKV_STATIC_SCRATCH_BYTES", "fa_bwd", "fa_bwd_workspace_bytes", "fwd_fp8_block", "quantize_e4m3_block", "fa_fwd", "fa_fwd_local", "fa_fwd_fp8_block",
           "fa_quantize_e4m3_block", "fa_fwd_query", "FP8_BLOCK_ROWS", "status_string", "version", "FaError", "FA_OK",
           "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_LAUNCH", "FA_DTYPE_F16", "FA_DTYPE_BF16",
           "FA_DTYPE_FP8_E4M3"]
