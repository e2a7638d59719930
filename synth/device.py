"""Placing seeded inputs on the GPU for the library's Python binding.

Plumbing only, no arithmetic of the method: a workload's sizes become the
binding's Problem descriptor, and stored host arrays (bf16 bit patterns or
float32) become device tensors with the same bits.  Kept apart from the
generator so that the oracle's tests never import torch's device code or the
binding through synth.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .latents import bf16_bits_to_f32
from .workloads import Workload


def problem_of(w: Workload, heads: Optional[int] = None):
    """The binding's Problem for workload ``w`` (optionally with another head count)."""
    import dynamic_sparse_attention_qk_amd as dsa
    return dsa.Problem(batch=w.batch, heads=w.heads if heads is None else heads, seq_len=w.seq_len,
                       head_dim=w.head_dim, rank=w.rank, group=w.group,
                       dtype=dsa.DSA_BF16 if w.dtype == "bf16" else dsa.DSA_F32)


def to_device(a: Optional[np.ndarray], device="cuda"):
    """A device tensor holding exactly the stored values of ``a`` (uint16 arrays are bf16 bit patterns)."""
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def f64(a: np.ndarray) -> np.ndarray:
    """Stored values lifted exactly to float64."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)
