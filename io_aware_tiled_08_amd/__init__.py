"""MI355X-native FlashAttention forward pass.

The computation runs in hand-written gfx950 HIP kernels inside
``libfa_mi355x.so`` (C ABI: include/fa_mi355x.h); this package only marshals
torch tensors into that ABI.
"""
from .binding import (FA_BF16, FA_F16, FA_F32, FlashAttnError, flash_attn_bwd, flash_attn_fwd,
                      flash_attn_fwd_fp8, flash_attn_fwd_kvcache, flash_attn_fwd_kvcache_noalloc,
                      flash_attn_fwd_kvcache_ptr,
                      flash_attn_fwd_persistent, flash_attn_fwd_persistent_ptr, flash_attn_fwd_ptr,
                      kvcache_splits, kvcache_workspace_size, last_error, lib)

__all__ = ["FA_BF16", "FA_F16", "FA_F32", "FlashAttnError", "flash_attn_bwd", "flash_attn_fwd",
           "flash_attn_fwd_fp8", "flash_attn_fwd_kvcache", "flash_attn_fwd_kvcache_noalloc",
           "flash_attn_fwd_kvcache_ptr",
           "flash_attn_fwd_persistent", "flash_attn_fwd_persistent_ptr", "flash_attn_fwd_ptr",
           "kvcache_splits", "kvcache_workspace_size", "last_error", "lib"]
