"""Fused scaled-dot-product attention forward for MI355X (gfx950)."""
