"""MI355X-native FlashAttention-2 forward and flash-decoding (placeholder; binding follows)."""
