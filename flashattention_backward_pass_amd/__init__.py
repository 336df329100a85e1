"""MI355X (gfx950) FlashAttention backward: Python binding of the C-ABI library."""
