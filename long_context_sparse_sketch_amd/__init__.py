"""Sparse-sketch long-context decode attention for MI355X (gfx950)."""
