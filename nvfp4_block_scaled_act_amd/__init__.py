"""NVFP4 quantized linear for MI355X (gfx950)."""
