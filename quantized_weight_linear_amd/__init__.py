"""Quantized-weight linear projection for AMD MI355X (gfx950)."""
