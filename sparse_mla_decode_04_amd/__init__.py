"""Sparse NVFP4 multi-head-latent-attention decode for MI355X (gfx950)."""
