"""Evoformer biased attention on MI355X (gfx950): fused HIP kernels behind a C ABI."""
