"""Paged decode attention and paged KV append for AMD Instinct MI355X (gfx950)."""
