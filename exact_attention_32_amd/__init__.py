"""MI355X (gfx950) fused exact-attention forward: Python binding over the C-ABI library."""
