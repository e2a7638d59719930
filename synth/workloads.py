"""The five seeded workloads, from a 1k-token fp32 forward to a 520k-token bf16 training step.

Each workload is a latent video grid (T x Y x X tokens), a head layout, the
predictor rank, the query-group size, the 64-token KV block and the number of
kept blocks per (head, query group).  The keep counts follow the plainest
reading of "keep a fraction f of NB blocks": k = clamp(floor(f*NB + 0.5), 1, NB)
(12.8 -> 13, 102.4 -> 102).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple


def keep_to_k(fraction: float, nb: int) -> int:
    """Kept-block count for a keep fraction: round half up, clamped to [1, nb]."""
    return int(min(max(math.floor(fraction * nb + 0.5), 1), nb))


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]          # (T, Y, X) latent grid; N = T*Y*X tokens
    n_centres: int                      # Voronoi cluster centres on the grid
    scale: Optional[float]              # cluster-vector scale; None -> per head U[scale_range]
    rank: int                           # predictor rank r
    group: int                          # query-group size G
    keep: Optional[float] = None        # uniform keep fraction of the NB blocks
    k: Optional[int] = None             # or an explicit uniform k
    keep_range: Optional[Tuple[float, float]] = None   # per head log-uniform keep fraction
    scale_range: Optional[Tuple[float, float]] = None  # per head uniform cluster scale
    dtype: str = "bf16"                 # storage dtype of Q, K, V, dO: "bf16" or "f32"
    backward: bool = True
    streamed: bool = False              # block scores streamed through the selection
    block: int = 64
    order: str = "morton"               # token order: "morton", or "cubes" (groups = aligned 4x4x(G/16) boxes)

    @property
    def seq_len(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block

    @property
    def n_groups(self) -> int:
        return self.seq_len // self.group

    def uniform_k(self) -> Optional[int]:
        if self.k is not None:
            return self.k
        if self.keep is not None:
            return keep_to_k(self.keep, self.n_blocks)
        return None

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload("tiny_fp32_fwd_1k", 1001, 1, 2, 64, (4, 16, 16), 8, 3.0, 16, 64,
                k=4, dtype="f32", backward=False),
    2: Workload("bf16_fwd_8k", 1002, 1, 16, 64, (8, 32, 32), 32, 3.0, 16, 64,
                keep=0.10, backward=False),
    3: Workload("bf16_train_57k", 1003, 1, 24, 128, (16, 45, 80), 64, 3.0, 32, 64,
                keep=0.10, backward=True),
    4: Workload("bf16_train_131k_g128", 1004, 1, 24, 128, (32, 64, 64), 128, 3.0, 32, 128,
                keep=0.05, backward=True),
    5: Workload("bf16_train_520k_imbalanced", 1005, 1, 24, 128, (40, 104, 125), 512, None, 32, 64,
                keep_range=(0.02, 0.30), scale_range=(1.5, 4.5), backward=True, streamed=True),
}


def workload(i: int) -> Workload:
    return WORKLOADS[i]
