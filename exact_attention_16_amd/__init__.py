"""MI355X-native exact-attention forward (FlashAttention-2 style) for gfx950."""
