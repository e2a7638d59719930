"""Seeded synthetic video-latent inputs shared by the tests, the bench and the oracle's tests.

This package holds no arithmetic of the sparse-attention method: it only draws
random tensors with a fixed recipe (Voronoi-clustered Q/K in a Morton- or cube-ordered
3D latent grid, Gaussian V and dO, Gaussian predictor weights) and rounds them
to the storage dtype.  Both the HIP path and the CPU oracle consume the exact
stored values it returns.
"""
from .workloads import WORKLOADS, Workload, keep_to_k, workload
from .latents import (Inputs, generate, bf16_bits_to_f32, f32_to_bf16_bits, random_dense, morton_order, cube_order,
                      cube_box, token_order, per_head_k)

__all__ = [
    "WORKLOADS", "Workload", "workload", "keep_to_k",
    "Inputs", "generate", "bf16_bits_to_f32", "f32_to_bf16_bits", "random_dense", "morton_order", "cube_order",
    "cube_box", "token_order", "per_head_k",
]
