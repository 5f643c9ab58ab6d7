"""Dropless MoE expert layer for MI355X (gfx950).

The device library (``libmoe.so``, hand-written HIP) is loaded on first use
by :mod:`dropless_moe_expert_amd.ops`; importing the package does not touch
the GPU.
"""
__all__ = ["inputs", "ops"]
