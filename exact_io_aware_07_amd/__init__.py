"""Exact IO-aware attention (forward and backward) for one MI355X (gfx950).

The computation lives in libfa.so (HIP kernels behind the C ABI of
include/fa.h); this package holds its ctypes binding, the in-tree build and
the seeded synthetic workloads.
"""
from .fa import (FA_BF16, FA_ERR_HIP, FA_ERR_INVALID_ARG, FA_ERR_TOO_LARGE, FA_ERR_UNSUPPORTED,
                 FA_ERR_WORKSPACE, FA_F16, FA_F32, FA_NOALLOC_MAX_ROWS, FA_OK, FaError,
                 attention_backward, attention_forward, fa_bwd, fa_bwd_noalloc,
                 fa_bwd_dkdv, fa_bwd_dq, fa_bwd_dsum, fa_bwd_gqa, fa_bwd_gqa_workspace_bytes,
                 fa_bwd_sparse, fa_bwd_sparse_planned, fa_bwd_sparse_planned_workspace_bytes,
                 fa_bwd_workspace_bytes, fa_fp8_quantize, fa_fwd, fa_fwd_fp8,
                 fa_fwd_fp8_incoherent, fa_fwd_fp8_workspace_bytes, fa_fwd_gqa, fa_fwd_partial,
                 fa_fwd_sparse, fa_fwd_split, fa_fwd_split_workspace_bytes, fa_merge,
                 fa_fwd_sparse_planned, fa_fwd_sparse_planned_workspace_bytes,
                 fa_sparse_plan, fa_strerror, fp8_buffers, lib, scaled_dot_product_attention)

__all__ = ["fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_noalloc", "fa_bwd_dsum", "fa_bwd_dkdv",
           "fa_bwd_dq", "fa_fwd_partial", "fa_merge", "fa_fwd_split_workspace_bytes",
           "fa_fwd_split", "fa_fwd_gqa", "fa_bwd_gqa_workspace_bytes", "fa_bwd_gqa", "fa_fwd_sparse",
           "fa_bwd_sparse", "fa_sparse_plan", "fa_fwd_sparse_planned_workspace_bytes",
           "fa_fwd_sparse_planned", "fa_bwd_sparse_planned_workspace_bytes",
           "fa_bwd_sparse_planned", "fa_fp8_quantize", "fa_fwd_fp8", "fa_fwd_fp8_workspace_bytes",
           "fa_fwd_fp8_incoherent", "fp8_buffers", "fa_strerror", "attention_forward",
           "attention_backward", "scaled_dot_product_attention", "lib", "FaError", "FA_F32", "FA_F16", "FA_BF16", "FA_OK",
           "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP",
           "FA_ERR_TOO_LARGE", "FA_NOALLOC_MAX_ROWS"]
