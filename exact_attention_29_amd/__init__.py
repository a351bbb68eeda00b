"""MI355X-native FlashAttention forward (placeholder; the binding lands with the kernel)."""
