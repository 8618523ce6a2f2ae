"""Exact attention forward for AMD MI355X (gfx950): Python binding placeholder."""
