"""Fused cross-entropy over a large vocabulary for AMD MI355X (gfx950)."""
