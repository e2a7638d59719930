"""Seeded generator of clustered video-latent Q/K/V/dO and predictor weights.

Recipe (everything derives from ``numpy.random.SeedSequence(workload.seed)``):

* Token order.  The T x Y x X latent grid is flattened in Morton (Z) order of
  (t, y, x): key = sum_b (t_b*4 + y_b*2 + x_b) * 8**b over the coordinate bits
  b, tokens sorted by key.  Consecutive runs of 64 tokens are then compact 3D
  neighbourhoods, the adjacency that query grouping relies on.  Option
  (``order="cubes"``): the aligned 4x4x(G/16) boxes that lie wholly inside the
  grid first (boxes in Morton order, cells in Morton order within each box),
  then the remaining cells in Morton order, so every group is one box.
* Structure stream (child 0 of the seed sequence), drawn in this order:
  cluster centres (distinct grid cells, uniform without replacement), one
  N(0, I_d) vector per (head, centre) (float64), then -- per-head workloads
  only -- the cluster scale s_h ~ U[lo, hi] for all heads and the keep fraction
  f_h = exp(U[ln lo, ln hi]) for all heads, then the predictor weight
  W ~ N(0, 1/d) of shape [H, d, r] (float64, rounded to float32).  The same W
  serves as W_q and W_k.
* Each token belongs to the nearest centre (squared Euclidean distance in grid
  index units, ties to the lowest centre id).
* Noise streams: child 1 + ((tensor * B + b) * H + h) for tensor 0..3 = Q, K,
  V, dO; each draws N(0, 1) float32 of shape [N, d].  Q and K get
  s_h * E[h, centre(token)] added in float32; V and dO get nothing.
* Storage: bf16 by round-to-nearest-even of the float32 value, or float32.

Returned tensors are [B, H, N, d] arrays of the stored values (uint16 bf16 bit
patterns or float32) -- the exact operands both implementations read.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from .workloads import Workload, keep_to_k


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def morton_order(grid) -> np.ndarray:
    """Grid cells (t, y, x) as an [N, 3] int64 array in Morton order."""
    t_n, y_n, x_n = grid
    t, y, x = np.meshgrid(np.arange(t_n), np.arange(y_n), np.arange(x_n), indexing="ij")
    t, y, x = t.ravel(), y.ravel(), x.ravel()
    key = np.zeros(t.shape, dtype=np.int64)
    nbits = int(max(t_n, y_n, x_n) - 1).bit_length() + 1
    for b in range(nbits):
        digit = ((t >> b) & 1) * 4 + ((y >> b) & 1) * 2 + ((x >> b) & 1)
        key |= digit.astype(np.int64) << (3 * b)
    order = np.argsort(key, kind="stable")
    return np.stack([t[order], y[order], x[order]], axis=1).astype(np.int64)


def _morton_keys(t: np.ndarray, y: np.ndarray, x: np.ndarray, nbits: int) -> np.ndarray:
    key = np.zeros(t.shape, dtype=np.int64)
    for b in range(nbits):
        digit = ((t >> b) & 1) * 4 + ((y >> b) & 1) * 2 + ((x >> b) & 1)
        key |= digit.astype(np.int64) << (3 * b)
    return key


def cube_box(group: int) -> Tuple[int, int, int]:
    """The (t, y, x) box one query group fills in cube order: 4x4x4 for 64 tokens, 4x4x8 for 128."""
    if group % 16 or group < 16:
        raise ValueError("cube order needs a group size that is a multiple of 16")
    return (4, 4, group // 16)


def cube_order(grid, group: int) -> np.ndarray:
    """Grid cells (t, y, x) as an [N, 3] int64 array in cube order for groups of ``group`` tokens.

    The grid is tiled by aligned boxes of cube_box(group) cells (a union of aligned 2x2x2 cubes).  The boxes
    that lie wholly inside the grid come first, in Morton order of their box coordinates, each box's cells in
    Morton order within it, so that every group of ``group`` consecutive tokens among them is exactly one box.
    The cells of the partial boxes along sides not divisible by the box follow, in Morton order of their grid
    coordinates.
    """
    t_n, y_n, x_n = grid
    bt, by, bx = cube_box(group)
    t, y, x = np.meshgrid(np.arange(t_n), np.arange(y_n), np.arange(x_n), indexing="ij")
    t, y, x = t.ravel(), y.ravel(), x.ravel()
    full = (t < (t_n // bt) * bt) & (y < (y_n // by) * by) & (x < (x_n // bx) * bx)
    nb = int(max(t_n, y_n, x_n) - 1).bit_length() + 1
    box_key = _morton_keys(t // bt, y // by, x // bx, nb)
    in_key = _morton_keys(t % bt, y % by, x % bx, 4)
    glob_key = _morton_keys(t, y, x, nb)
    # full boxes first (by box, then within the box), then the partial-box cells by their own Morton key
    order = np.lexsort((np.where(full, in_key, glob_key), np.where(full, box_key, 0), ~full))
    return np.stack([t[order], y[order], x[order]], axis=1).astype(np.int64)


def token_order(w: Workload) -> np.ndarray:
    """The workload's token order: ``w.order`` "morton" (default) or "cubes"."""
    if w.order == "morton":
        return morton_order(w.grid)
    if w.order == "cubes":
        return cube_order(w.grid, w.group)
    raise ValueError(f"unknown token order {w.order!r}")


def nearest_centre(coords: np.ndarray, centres: np.ndarray, chunk: int = 65536) -> np.ndarray:
    """Index of the nearest centre for each coordinate (exact integer distances, lowest id on ties)."""
    out = np.empty(coords.shape[0], dtype=np.int64)
    for s in range(0, coords.shape[0], chunk):
        c = coords[s:s + chunk]
        d2 = ((c[:, None, :] - centres[None, :, :]) ** 2).sum(axis=2)
        out[s:s + chunk] = np.argmin(d2, axis=1)
    return out


@dataclass
class Inputs:
    workload: Workload
    q: np.ndarray                 # [B, H, N, d] uint16 (bf16 bits) or float32
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    w: np.ndarray                 # [H, d, r] float32 (W_q = W_k)
    k_per_head: np.ndarray        # [H] int32 kept blocks per (head, group)
    coords: np.ndarray            # [N, 3] token grid coordinates (in the workload's token order)
    cell_centre: np.ndarray       # [N] nearest-centre id of each token
    head_scale: np.ndarray        # [H] cluster scale per head
    head_keep: np.ndarray         # [H] keep fraction per head (nan when k is explicit)

    @property
    def is_bf16(self) -> bool:
        return self.workload.dtype == "bf16"

    def as_f64(self, name: str) -> np.ndarray:
        """Stored values of a tensor lifted exactly to float64."""
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def _structure(w: Workload, rng: np.random.Generator, coords: np.ndarray):
    ncell = coords.shape[0]
    cid = rng.choice(ncell, size=w.n_centres, replace=False)
    centres = coords[cid]
    emb = rng.standard_normal((w.heads, w.n_centres, w.head_dim))
    if w.scale_range is not None:
        lo, hi = w.scale_range
        scale = rng.uniform(lo, hi, size=w.heads)
    else:
        scale = np.full(w.heads, float(w.scale))
    if w.keep_range is not None:
        lo, hi = w.keep_range
        keep = np.exp(rng.uniform(np.log(lo), np.log(hi), size=w.heads))
        kph = np.array([keep_to_k(f, w.n_blocks) for f in keep], dtype=np.int32)
    else:
        keep = np.full(w.heads, np.nan if w.keep is None else float(w.keep))
        kph = np.full(w.heads, w.uniform_k(), dtype=np.int32)
    wts = (rng.standard_normal((w.heads, w.head_dim, w.rank)) * np.sqrt(1.0 / w.head_dim)).astype(np.float32)
    return centres, emb, scale, keep, kph, wts


def generate(w: Workload, threads: int = 8, heads: Optional[Sequence[int]] = None) -> Inputs:
    """Draw the inputs of workload ``w`` (deterministic for a given workload).

    ``heads`` restricts the draw to a subset of heads; each drawn head holds
    exactly the values the full draw gives it (per-head streams).
    """
    if w.seq_len % w.block or w.seq_len % w.group:
        raise ValueError("token count must be a multiple of the block and group sizes")
    coords = token_order(w)
    root = np.random.SeedSequence(w.seed)
    n_tensors = 4 if w.backward else 3
    children = root.spawn(1 + n_tensors * w.batch * w.heads)
    centres, emb, scale, keep, kph, wts = _structure(w, np.random.Generator(np.random.PCG64(children[0])), coords)
    owner = nearest_centre(coords, centres)

    n, d = w.seq_len, w.head_dim
    hsel = list(range(w.heads)) if heads is None else [int(h) for h in heads]
    store = np.uint16 if w.dtype == "bf16" else np.float32
    shape = (w.batch, len(hsel), n, d)
    outs = [np.empty(shape, dtype=store) for _ in range(n_tensors)]

    def fill(job):
        t, b, hi = job
        h = hsel[hi]
        rng = np.random.Generator(np.random.PCG64(children[1 + (t * w.batch + b) * w.heads + h]))
        x = rng.standard_normal((n, d), dtype=np.float32)
        if t < 2:
            x += (scale[h] * emb[h]).astype(np.float32)[owner]
        outs[t][b, hi] = f32_to_bf16_bits(x) if w.dtype == "bf16" else x

    jobs = [(t, b, hi) for t in range(n_tensors) for b in range(w.batch) for hi in range(len(hsel))]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, jobs))

    return Inputs(
        workload=w, q=outs[0], k=outs[1], v=outs[2], do=outs[3] if w.backward else None,
        w=wts[hsel], k_per_head=kph[hsel], coords=coords, cell_centre=owner, head_scale=scale[hsel],
        head_keep=keep[hsel],
    )


def per_head_k(w: Workload) -> np.ndarray:
    """The kept-block counts k_h of a workload without drawing its tensors."""
    coords = token_order(w)
    child = np.random.SeedSequence(w.seed).spawn(1)[0]
    return _structure(w, np.random.Generator(np.random.PCG64(child)), coords)[4]


def random_dense(shape, seed: int, dtype: str = "bf16", scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) tensor in storage dtype, for shape sweeps and edge cases."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def as_dict(inp: Inputs) -> Dict[str, np.ndarray]:
    return {"q": inp.q, "k": inp.k, "v": inp.v, "do": inp.do, "w": inp.w, "k_per_head": inp.k_per_head}
