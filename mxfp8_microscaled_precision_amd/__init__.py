"""MXFP8 microscaled-precision hot path for MI355X (gfx950)."""
