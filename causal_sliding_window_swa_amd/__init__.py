"""Causal sliding-window attention for MI355X (gfx950)."""
