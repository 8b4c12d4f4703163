"""MI355X (gfx950) fused multi-head attention backward."""
