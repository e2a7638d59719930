"""Brute-force references used to pin the oracle on tiny inputs.

Written independently of oracle/: dense N x N matrices, explicit masks and
Python-level sorts, no pooling shortcuts.  Only for N of a few hundred.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import softmax


def tile_mean_scores(q, k, wq, wk, group, block=64):
    """Block scores from the full predicted-logit matrix, averaged over each G x Bk tile."""
    n, d = q.shape
    pred = ((q @ wq) @ (k @ wk).T) / math.sqrt(d)           # N x N predicted logits
    ng, nb = n // group, n // block
    out = np.empty((ng, nb))
    for g in range(ng):
        for j in range(nb):
            out[g, j] = pred[g * group:(g + 1) * group, j * block:(j + 1) * block].sum() / (group * block)
    return out


def true_tile_mean(q, k, group, block=64):
    """Tile means of the true attention logits tau Q K^T."""
    n, d = q.shape
    lg = (q @ k.T) / math.sqrt(d)
    return np.array([[lg[g * group:(g + 1) * group, j * block:(j + 1) * block].mean()
                      for j in range(n // block)] for g in range(n // group)])


def topk_sorted(row, k):
    """Python sort of (-s, j) tuples; first k ids, ascending."""
    pairs = sorted(((-float(s), j) for j, s in enumerate(row)))
    return sorted(j for _, j in pairs[:k])


def mask_from_idx(idx_bh, n, group, block=64):
    """Boolean N x N mask: query i may see key m iff m's block is kept by i's group."""
    mask = np.zeros((n, n), dtype=bool)
    for g in range(n // group):
        for j in idx_bh[g]:
            mask[g * group:(g + 1) * group, int(j) * block:(int(j) + 1) * block] = True
    return mask


def masked_attention(q, k, v, mask):
    """Dense masked softmax attention: O, LSE (direct log-sum-exp, no max shift), P."""
    d = q.shape[1]
    lg = (q @ k.T) / math.sqrt(d)
    lg = np.where(mask, lg, -np.inf)
    p = softmax(lg, axis=1)
    lse = np.log(np.where(mask, np.exp(np.where(mask, lg, 0.0)), 0.0).sum(axis=1))
    return p @ v, lse, p


def finite_diff_grads(q, k, v, do, mask, h=1e-6):
    """Central differences of L = sum(dO * O) w.r.t. every entry of Q, K, V."""
    def loss(qq, kk, vv):
        return float((do * masked_attention(qq, kk, vv, mask)[0]).sum())

    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][ix] += h
            minus[which][ix] -= h
            g[ix] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads
