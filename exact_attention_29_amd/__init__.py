"""MI355X-native FlashAttention forward pass and its gradients.

    from exact_attention_29_amd import attention, attention_bwd
    o, lse = attention(q, k, v, causal=False, scale=None)
    dq, dk, dv = attention_bwd(q, k, v, o, lse, dout, causal=False, scale=None)

q, k, v are contiguous device tensors [B, H, N, d] (bf16, fp16 or fp32).  All
arithmetic runs in the HIP kernels of libfa.so behind the C ABI of
include/fa.h; this package only marshals arguments.  There is no CPU path:
without the built library every call raises.
"""
from ._native import (FA_DTYPE_BF16, FA_DTYPE_FP16, FA_DTYPE_FP32, FA_ERR_HIP,
                      FA_ERR_INVALID_ARG, FA_ERR_SCRATCH, FA_ERR_UNSUPPORTED,
                      FA_NOALLOC_SCRATCH_BYTES, FA_OK, FaError,
                      attention, attention_bwd, fa_bwd, fa_bwd_ex, fa_bwd_ex_workspace_size,
                      fa_bwd_gen, fa_bwd_gen_supported, fa_bwd_gen_workspace_size,
                      fa_bwd_supported,
                      fa_bwd_workspace_size, fa_fwd, fa_fwd_ex, fa_fwd_ex_workspace_size,
                      fa_fwd_gen, fa_fwd_gen_noalloc, fa_fwd_gen_supported,
                      fa_fwd_gen_workspace_size,
                      fa_fwd_supported, fa_fwd_workspace_size,
                      fa_fwd_ws, fa_status_string, fa_version, library, library_path)

__all__ = ["attention", "attention_bwd", "fa_bwd", "fa_bwd_ex", "fa_bwd_ex_workspace_size",
           "fa_bwd_gen", "fa_bwd_gen_supported", "fa_bwd_gen_workspace_size", "fa_bwd_supported",
           "fa_bwd_workspace_size",
           "fa_fwd", "fa_fwd_ex", "fa_fwd_ex_workspace_size", "fa_fwd_gen", "fa_fwd_gen_noalloc", "fa_fwd_gen_supported",
           "fa_fwd_gen_workspace_size", "fa_fwd_ws", "fa_fwd_workspace_size", "fa_fwd_supported",
           "fa_status_string", "fa_version",
           "library", "library_path", "FaError", "FA_OK", "FA_ERR_INVALID_ARG",
           "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_ERR_SCRATCH", "FA_NOALLOC_SCRATCH_BYTES", "FA_DTYPE_FP32", "FA_DTYPE_FP16",
           "FA_DTYPE_BF16"]
