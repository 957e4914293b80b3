"""Paged-attention decode for MI355X (gfx950)."""
