"""Blockwise ring-attention step for AMD MI355X (gfx950)."""
