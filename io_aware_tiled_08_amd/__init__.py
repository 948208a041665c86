"""MI355X-native FlashAttention forward pass (gfx950 HIP kernels behind a C ABI)."""
