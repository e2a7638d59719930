"""Plain float64 CPU oracle of DSV's sparse-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, links or calls this module; only the tests, the smoke
check and the bench's CPU-baseline leg do.  It shares no code with the HIP path.

Source pages: the gist.science explainers (Dutch "nl" and Hindi "hi" editions)
of "DSV: Exploiting Dynamic Sparsity to Accelerate Large-Scale Video DiT
Training", cited below by edition and technical-summary section.

What is computed, per batch b and head h, on the exact stored input values
lifted to float64 (tau = 1/sqrt(d), Bk = 64-token KV blocks, G-token query
groups of consecutive tokens):

1. pooled proxy query of each group and pooled key of each block (mean);
2. low-rank projection through the per-head predictor weights W_q, W_k
   (d x r, r << d)                                   [hi §2.A, nl §2.A]
3. block score s[g, j] = tau * qhat_g . khat_j -- the predictor's estimate of
   the group-to-block attention logits              [hi §2.A, §2.B query grouping]
   (a variant pools the token-level predicted logits of each G x 64 tile by
   max or by log-mean-exp instead of pooling Q and K first)
4. per group, the k_h blocks of largest score, ties to the lowest block id,
   listed ascending -- the "critical" KV blocks     [hi §2.A, §2.B fused MM + top-k]
   or, by coverage, the shortest run of blocks in score order whose estimated
   attention mass (softmax of the block scores) reaches a fraction, capped
   per head (rows then differ in length)            [hi §2.A critical KV ~90%]
   and, in either rule, optionally with the blocks that hold the group's own
   tokens always kept (a forced diagonal; a variant, not from the pages)
5. exact softmax attention of every query of the group over the keys of its
   kept blocks only (no mask beyond the selection; bidirectional)
                                                    [hi §2.A stage 2, nl §2.A fase 2]
   and split-KV partial states over parts of the kept list with their merge
   (LSE = logsumexp of the parts' LSE, O their exp-weighted sum)
                                                    [DiTango nl Methodologie; hi §2.C]
   and, for the OP dispatcher's other branch, full (dense) attention over all
   keys, with the dispatcher's rule: sparse iff the skipped fraction of
   (head, group, block) tiles exceeds a threshold   [hi §2.A, nl §2.A stage 2]
6. the gradient of L = sum(dO * O) with the selection held fixed: dQ, dK, dV
   (keys in no kept block get exactly zero).  The pages call the method a
   training system but never write the backward out; this is the standard
   softmax-attention gradient restricted to the kept keys.
7. stage-1 predictor training: a loss on the row-centred difference between
   the block scores and the true pooled logits, and its gradient with respect
   to W_q and W_k                                    [hi §2.A, nl §2.A stage 1]

Every function here is pinned by tests/test_oracle.py against brute force on
tiny inputs, a library routine (torch's scaled_dot_product_attention and
autograd), central finite differences, closed forms and invariants.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

BLOCK = 64


# ----------------------------------------------------------------------------
# Steps 1-3: predictor (pooling, projection, block scores)
# ----------------------------------------------------------------------------

def pool_mean(x: np.ndarray, size: int) -> np.ndarray:
    """Mean over consecutive runs of ``size`` rows: [n, d] -> [n / size, d].

    The proxy query of a query group is the group's centroid, and a KV block is
    represented by its mean key (hi §2.B query grouping: one proxy per group
    whose critical indices the whole group reuses).
    """
    n, d = x.shape
    assert n % size == 0
    return x.reshape(n // size, size, d).mean(axis=1)


def predict_head(q: np.ndarray, k: np.ndarray, wq: np.ndarray, wk: np.ndarray,
                 group: int, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Low-rank block-score estimate for one (b, h): returns (qhat, khat, scores).

    qhat = pool(Q) W_q [NG, r], khat = pool(K) W_k [NB, r], scores = tau qhat khat^T
    [NG, NB], tau = 1/sqrt(d) with d the head dimension (hi §2.A: predictors
    W^Q_lr, W^K_lr estimate QK^T through a d_lr << d_k projection).
    """
    d = q.shape[1]
    tau = 1.0 / np.sqrt(d)
    qhat = pool_mean(q, group) @ wq
    khat = pool_mean(k, block) @ wk
    return qhat, khat, tau * (qhat @ khat.T)


def predict(q: np.ndarray, k: np.ndarray, wq: np.ndarray, wk: np.ndarray,
            group: int, block: int = BLOCK):
    """predict_head over [B, H, N, d] inputs and [H, d, r] weights."""
    B, H = q.shape[:2]
    out = [[predict_head(q[b, h], k[b, h], wq[h], wk[h], group, block) for h in range(H)] for b in range(B)]
    qhat = np.stack([np.stack([o[0] for o in row]) for row in out])
    khat = np.stack([np.stack([o[1] for o in row]) for row in out])
    scores = np.stack([np.stack([o[2] for o in row]) for row in out])
    return qhat, khat, scores


def predict_head_pooled(q: np.ndarray, k: np.ndarray, wq: np.ndarray, wk: np.ndarray, group: int, pooling: str,
                        block: int = BLOCK) -> np.ndarray:
    """Block scores pooled from the token-level predicted logits l[i, m] = tau (q_i W_q) . (k_m W_k) over each
    G x 64 tile, a predictor variant: "mean" (equal to predict_head's scores), "max" (the tile's largest
    logit), or "lse" (log of the tile's mean of exp(l): the log of the predicted attention mass per key pair,
    so that exp(score) ranks blocks by their predicted share of the softmax)."""
    n, d = q.shape
    tau = 1.0 / np.sqrt(d)
    lg = tau * ((q @ wq) @ (k @ wk).T)                              # N x N predicted logits
    t = lg.reshape(n // group, group, n // block, block)           # [g, i, j, m]
    if pooling == "mean":
        return t.mean(axis=(1, 3))
    if pooling == "max":
        return t.max(axis=(1, 3))
    if pooling == "lse":
        m = t.max(axis=(1, 3), keepdims=True)
        return (m + np.log(np.exp(t - m).mean(axis=(1, 3), keepdims=True)))[:, 0, :, 0]
    raise ValueError(pooling)


def predict_head_pooled_groups(q, k, wq, wk, group, pooling, groups, block=BLOCK) -> Dict[int, np.ndarray]:
    """Rows of predict_head_pooled for the listed groups only (the same arithmetic on their query rows)."""
    out = {}
    for g in groups:
        rows = slice(g * group, (g + 1) * group)
        # the group's rows against every key: one [1, NB] row of the pooled scores
        out[g] = predict_head_pooled_rows(q[rows], k, wq, wk, pooling, block)
    return out


def predict_head_pooled_rows(qg, k, wq, wk, pooling, block=BLOCK) -> np.ndarray:
    tau = 1.0 / np.sqrt(qg.shape[1])
    lg = tau * ((qg @ wq) @ (k @ wk).T)                                # G x N predicted logits
    t = lg.reshape(qg.shape[0], k.shape[0] // block, block)             # [i, j, m]
    if pooling == "mean":
        return t.mean(axis=(0, 2))
    if pooling == "max":
        return t.max(axis=(0, 2))
    if pooling == "lse":
        m = t.max(axis=(0, 2), keepdims=True)
        return (m + np.log(np.exp(t - m).mean(axis=(0, 2), keepdims=True)))[0, :, 0]
    raise ValueError(pooling)


# ----------------------------------------------------------------------------
# Step 4: top-k critical block selection
# ----------------------------------------------------------------------------

def select_row(scores_row: np.ndarray, k: int) -> np.ndarray:
    """The k block ids of largest score, ties to the lowest id, returned ascending.

    Sorting the pairs (-s_j, j) lexicographically and keeping the first k is the
    definition; -0.0 and +0.0 compare equal, as IEEE equality says (hi §2.A
    critical KV estimation, §2.B top-k selection).
    """
    nb = scores_row.shape[0]
    assert 1 <= k <= nb
    s = np.asarray(scores_row)
    order = np.lexsort((np.arange(nb), -s))      # primary key -s, secondary key j
    return np.sort(order[:k]).astype(np.int64)


def select_rows(scores: np.ndarray, k: int) -> np.ndarray:
    """select_row for every row of an [NG, NB] score matrix at once: [NG, k] ascending ids.

    The same definition (order by -s, ties to the lowest id, keep the first k): a stable sort of -s keeps
    equal scores in id order, and -0.0, +0.0 compare equal in it.
    """
    s = np.asarray(scores)
    nb = s.shape[1]
    assert 1 <= k <= nb
    order = np.argsort(-s, axis=1, kind="stable")[:, :k]
    return np.sort(order, axis=1).astype(np.int64)


def diagonal_blocks(g: int, group: int, n_blocks: int, block: int = BLOCK) -> np.ndarray:
    """The KV blocks that hold query group g's own tokens."""
    return np.arange(g * group // block, min((g + 1) * group // block, n_blocks))


def select_order(scores_row: np.ndarray, forced: Sequence[int] = ()) -> np.ndarray:
    """Blocks in selection order: the forced ones first (ascending), then the rest by decreasing score,
    ties to the lowest id."""
    nb = len(scores_row)
    s = np.asarray(scores_row)
    order = np.lexsort((np.arange(nb), -s))
    f = np.asarray(sorted(int(j) for j in forced), dtype=np.int64)
    return np.concatenate([f, order[~np.isin(order, f)]]).astype(np.int64)


def select_row_diag(scores_row: np.ndarray, k: int, g: int, group: int, block: int = BLOCK) -> np.ndarray:
    """Top-k with the group's own blocks always kept (k at least their number): the first k blocks of
    select_order with those blocks forced, ascending."""
    forced = diagonal_blocks(g, group, len(scores_row), block)
    assert len(forced) <= k <= len(scores_row)
    return np.sort(select_order(scores_row, forced)[:k])


def select_coverage_row_diag(scores_row: np.ndarray, coverage: float, k_cap: int, g: int, group: int,
                             block: int = BLOCK) -> np.ndarray:
    """Coverage selection whose run starts with the group's own blocks (always kept, their estimated mass
    counted), then the rest in score order; at most k_cap blocks (k_cap at least the forced count)."""
    forced = diagonal_blocks(g, group, len(scores_row), block)
    order = select_order(scores_row, forced)
    cum = np.cumsum(block_mass(scores_row)[order])
    c = max(len(forced), 1 + int(np.count_nonzero(cum < coverage)))
    return np.sort(order[:min(c, k_cap, len(scores_row))])


def select(scores: np.ndarray, k_per_head: Sequence[int]) -> List[List[np.ndarray]]:
    """Per (b, h): an [NG, k_h] array of ascending kept block ids."""
    B, H, NG, _ = scores.shape
    return [[np.stack([select_row(scores[b, h, g], int(k_per_head[h])) for g in range(NG)])
             for h in range(H)] for b in range(B)]


def reverse_index(idx_bh, n_blocks: int) -> List[np.ndarray]:
    """For each KV block j, the ascending list of query groups whose selection holds j (rows may differ in
    length)."""
    lists: List[List[int]] = [[] for _ in range(n_blocks)]
    for g in range(len(idx_bh)):
        for j in idx_bh[g]:
            lists[int(j)].append(g)
    return [np.asarray(l, dtype=np.int64) for l in lists]


def reverse_index_csr(idx_bh: np.ndarray, n_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
    """reverse_index of an [NG, k] list array in compressed form: (ptr [NB + 1], groups), block j's groups
    being groups[ptr[j]:ptr[j + 1]], ascending.  The (block, group) pairs are read row by row, i.e. in
    ascending group order, and stably sorted by block."""
    a = np.asarray(idx_bh, dtype=np.int64)
    ng, kk = a.shape
    flat = a.ravel()
    groups = np.repeat(np.arange(ng, dtype=np.int64), kk)
    order = np.argsort(flat, kind="stable")
    ptr = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=n_blocks))]).astype(np.int64)
    return ptr, groups[order]


def reverse_list(idx_bh: np.ndarray, j: int) -> np.ndarray:
    """Ascending query groups whose selection holds block j (one entry of reverse_index)."""
    return np.nonzero((np.asarray(idx_bh) == j).any(axis=1))[0].astype(np.int64)


def block_mass(scores_row: np.ndarray) -> np.ndarray:
    """Estimated share of a query's attention that falls in each KV block: every block holds 64 keys and
    its score estimates their mean logit, so the shares are the softmax of the row's block scores."""
    s = np.asarray(scores_row, dtype=np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def select_coverage_row(scores_row: np.ndarray, coverage: float, k_cap: int) -> np.ndarray:
    """The critical blocks by attention coverage (hi §2.A: the critical KV pairs are those that carry about
    90% of the attention score): in the order of decreasing score (ties to the lowest id), the shortest
    prefix whose estimated mass reaches ``coverage`` (0 < coverage <= 1), at most ``k_cap`` blocks;
    returned ascending."""
    nb = len(scores_row)
    s = np.asarray(scores_row)
    order = np.lexsort((np.arange(nb), -s))
    cum = np.cumsum(block_mass(s)[order])
    c = 1 + int(np.count_nonzero(cum < coverage))
    return np.sort(order[:min(c, k_cap, nb)]).astype(np.int64)


def select_coverage(scores: np.ndarray, coverage: float, k_cap_per_head: Sequence[int]):
    """Per (b, h): a list of NG ascending arrays (lengths vary by row)."""
    B, H, NG, _ = scores.shape
    return [[[select_coverage_row(scores[b, h, g], coverage, int(k_cap_per_head[h])) for g in range(NG)]
             for h in range(H)] for b in range(B)]


def kept_keys(idx_row: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Key positions covered by the kept blocks of one group, ascending."""
    return (np.asarray(idx_row, dtype=np.int64)[:, None] * block + np.arange(block)[None, :]).ravel()


# ----------------------------------------------------------------------------
# Step 5: exact attention over the kept keys
# ----------------------------------------------------------------------------

def group_forward(qg: np.ndarray, k: np.ndarray, v: np.ndarray, keys: np.ndarray):
    """Softmax attention of the rows of one group over ``keys`` only.

    logits l = tau q k^T; M = row max; LSE = M + ln sum exp(l - M);
    P = exp(l - LSE); O = P V.  Returns (O [G, d], LSE [G], P [G, |keys|]).
    """
    tau = 1.0 / np.sqrt(qg.shape[1])
    logits = tau * (qg @ k[keys].T)
    m = logits.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(logits - m).sum(axis=1))
    p = np.exp(logits - lse[:, None])
    return p @ v[keys], lse, p


def forward_head(q, k, v, idx_bh, group, block=BLOCK, groups=None):
    """O [N, d] and LSE [N] of one (b, h); with ``groups`` only those groups' rows are filled (rest NaN)."""
    n, d = q.shape
    o = np.full((n, d), np.nan)
    lse = np.full(n, np.nan)
    for g in (range(n // group) if groups is None else groups):
        rows = slice(g * group, (g + 1) * group)
        o[rows], lse[rows], _ = group_forward(q[rows], k, v, kept_keys(idx_bh[g], block))
    return o, lse


def forward(q, k, v, idx, group, block=BLOCK):
    """O [B, H, N, d] and LSE [B, H, N] for per-(b, h) selections ``idx[b][h]``."""
    B, H = q.shape[:2]
    o = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], idx[b][h], group, block)
    return o, lse


# ----------------------------------------------------------------------------
# Split-KV: partial attention states over parts of a row's kept blocks, merged
# (DiTango explainer, nl edition, technical summary, Methodologie: attention
# states -- output and log-sum-exp -- compose associatively and commutatively;
# DSV hi §2.C sparse sequence-wise CP: a device attends to the critical KV it
# holds)
# ----------------------------------------------------------------------------

def split_bounds(k: int, n_split: int) -> List[Tuple[int, int]]:
    """Positions [floor(s k / n), floor((s + 1) k / n)) of part s of a k-entry kept list."""
    return [(s * k // n_split, (s + 1) * k // n_split) for s in range(n_split)]


def partial_state(qg: np.ndarray, k: np.ndarray, v: np.ndarray, keys: np.ndarray):
    """(O_p, LSE_p) of the rows of one group over a subset ``keys`` of its kept keys: the softmax
    normalised within the subset.  An empty subset gives O_p = 0 and LSE_p = -inf."""
    if len(keys) == 0:
        return np.zeros((qg.shape[0], v.shape[1])), np.full(qg.shape[0], -np.inf)
    o, lse, _ = group_forward(qg, k, v, keys)
    return o, lse


def merge_states(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """LSE = ln sum_p exp(LSE_p); O = sum_p exp(LSE_p - LSE) O_p (a part with LSE_p = -inf adds nothing)."""
    lse_parts = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])
    m = lse_parts.max(axis=0)
    lse = m + np.log(np.exp(lse_parts - m).sum(axis=0))
    o = np.zeros_like(np.asarray(o_parts[0], dtype=np.float64))
    for op, lp in zip(o_parts, lse_parts):
        o = o + np.exp(lp - lse)[..., None] * op
    return o, lse


def forward_split_head(q, k, v, idx_bh, group, n_split, block=BLOCK, groups=None):
    """Per part s: O_s [N, d], LSE_s [N] of one (b, h) over part s of every group's kept list
    (only ``groups`` filled when given, the rest NaN)."""
    n, d = q.shape
    o = np.full((n_split, n, d), np.nan)
    lse = np.full((n_split, n), np.nan)
    for g in (range(n // group) if groups is None else groups):
        rows = slice(g * group, (g + 1) * group)
        row = np.asarray(idx_bh[g])
        for s, (a, e) in enumerate(split_bounds(len(row), n_split)):
            o[s, rows], lse[s, rows] = partial_state(q[rows], k, v, kept_keys(row[a:e], block))
    return o, lse


# ----------------------------------------------------------------------------
# Step 6: gradients with the selection held fixed
# ----------------------------------------------------------------------------

def group_backward(qg, k, v, dog, keys):
    """Gradient contributions of one group.

    With P and O from group_forward: D_i = sum_c dO_ic O_ic, dP = dO V^T,
    dS = P (dP - D), dQ_g = tau dS K, and the key-side terms
    dK[keys] += tau dS^T Q_g, dV[keys] += P^T dO_g.
    Returns (dQ_g, dK_part, dV_part, O_g, LSE_g).
    """
    tau = 1.0 / np.sqrt(qg.shape[1])
    og, lse, p = group_forward(qg, k, v, keys)
    dvec = (dog * og).sum(axis=1)
    dp = dog @ v[keys].T
    ds = p * (dp - dvec[:, None])
    return tau * (ds @ k[keys]), tau * (ds.T @ qg), p.T @ dog, og, lse


def backward_head(q, k, v, do, idx_bh, group, block=BLOCK):
    """dQ, dK, dV [N, d] of one (b, h) for L = sum(dO * O)."""
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for g in range(n // group):
        rows = slice(g * group, (g + 1) * group)
        keys = kept_keys(idx_bh[g], block)
        dq_g, dk_p, dv_p, _, _ = group_backward(q[rows], k, v, do[rows], keys)
        dq[rows] = dq_g
        dk[keys] += dk_p
        dv[keys] += dv_p
    return dq, dk, dv


def backward(q, k, v, do, idx, group, block=BLOCK):
    B, H = q.shape[:2]
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], idx[b][h], group, block)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Sampled evaluation for full-size workloads (same arithmetic, fewer outputs)
# ----------------------------------------------------------------------------

def dq_groups(q, k, v, do, idx_bh, group, groups, block=BLOCK) -> Dict[int, np.ndarray]:
    """dQ rows of the listed groups of one (b, h)."""
    out = {}
    for g in groups:
        rows = slice(g * group, (g + 1) * group)
        out[g] = group_backward(q[rows], k, v, do[rows], kept_keys(idx_bh[g], block))[0]
    return out


def dkdv_blocks(q, k, v, do, idx_bh, group, blocks, block=BLOCK) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
    """dK, dV rows of the listed KV blocks of one (b, h), summed over every group that kept them."""
    rev = reverse_index(idx_bh, k.shape[0] // block)
    out = {}
    for j in blocks:
        dk = np.zeros((block, k.shape[1]))
        dv = np.zeros((block, v.shape[1]))
        for g in rev[j]:
            rows = slice(g * group, (g + 1) * group)
            keys = kept_keys(idx_bh[g], block)
            _, dk_p, dv_p, _, _ = group_backward(q[rows], k, v, do[rows], keys)
            pos = int(np.searchsorted(idx_bh[g], j)) * block
            dk += dk_p[pos:pos + block]
            dv += dv_p[pos:pos + block]
        out[j] = (dk, dv)
    return out


def dkdv_block_part(q, k, v, do, idx_row, group, g, j, block=BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """What query group g adds to the dK and dV rows of KV block j (a block of g's kept list ``idx_row``):
    the group's softmax over all its kept keys gives LSE and O, hence D = dO . O; then on block j's keys only
    P = exp(tau q k^T - LSE), dS = P (dO v^T - D), dK_j += tau dS^T Q_g, dV_j += P^T dO_g.  Summed over the
    groups of block j's reverse list this is dkdv_blocks' result; one group at a time, so a caller can spread
    the groups of a long list over threads."""
    tau = 1.0 / np.sqrt(q.shape[1])
    rows = slice(g * group, (g + 1) * group)
    qg, dog = q[rows], do[rows]
    og, lse, _ = group_forward(qg, k, v, kept_keys(idx_row, block))
    dvec = (dog * og).sum(axis=1)
    kj, vj = k[j * block:(j + 1) * block], v[j * block:(j + 1) * block]
    p = np.exp(tau * (qg @ kj.T) - lse[:, None])
    ds = p * (dog @ vj.T - dvec[:, None])
    return tau * (ds.T @ qg), p.T @ dog


# ----------------------------------------------------------------------------
# Dense attention and the OP dispatcher (hi and nl §2.A, stage 2: per
# transformer block, sparse attention is switched on only when the block's
# sparsity exceeds a threshold found by offline profiling; below it the block
# keeps full attention, as in stage 1)
# ----------------------------------------------------------------------------

def dense_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray):
    """O [r, d] and LSE [r] of the given query rows over ALL keys: O = softmax(tau q K^T) V,
    LSE = ln sum_m exp(tau q . k_m).  Every row is independent of the others."""
    tau = 1.0 / np.sqrt(q_rows.shape[1])
    logits = tau * (q_rows @ k.T)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    l = w.sum(axis=1)
    return (w @ v) / l[:, None], m[:, 0] + np.log(l)


def dense_forward_head(q, k, v):
    """O [N, d], LSE [N] of full attention for one (b, h)."""
    return dense_rows(q, k, v)


def dense_backward_head(q, k, v, do):
    """dQ, dK, dV [N, d] of L = sum(dO * O) for full attention of one (b, h):
    P = exp(tau Q K^T - LSE), D_i = dO_i . O_i, dS = P (dO V^T - D),
    dQ = tau dS K, dK = tau dS^T Q, dV = P^T dO."""
    tau = 1.0 / np.sqrt(q.shape[1])
    o, lse = dense_rows(q, k, v)
    p = np.exp(tau * (q @ k.T) - lse[:, None])
    ds = p * (do @ v.T - (do * o).sum(axis=1)[:, None])
    return tau * (ds @ k), tau * (ds.T @ q), p.T @ do


def dense_forward(q, k, v):
    """O [B, H, N, d] and LSE [B, H, N] of full attention."""
    o = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty(q.shape[:3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            o[b, h], lse[b, h] = dense_forward_head(q[b, h], k[b, h], v[b, h])
    return o, lse


def dense_backward(q, k, v, do):
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            dq[b, h], dk[b, h], dv[b, h] = dense_backward_head(q[b, h], k[b, h], v[b, h], do[b, h])
    return dq, dk, dv


def dense_dq_rows(q, k, v, do, rows) -> np.ndarray:
    """dQ of the listed query rows of one (b, h) under full attention (one row needs only its own P)."""
    tau = 1.0 / np.sqrt(q.shape[1])
    qr, dor = q[rows], do[rows]
    o, lse = dense_rows(qr, k, v)
    p = np.exp(tau * (qr @ k.T) - lse[:, None])
    ds = p * (dor @ v.T - (dor * o).sum(axis=1)[:, None])
    return tau * (ds @ k)


def dense_dkdv_blocks(q, k, v, do, blocks, block=BLOCK, chunk=2048) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
    """dK, dV rows of the listed 64-key blocks of one (b, h) under full attention: the sums over
    every query i of tau dS_im q_i and P_im dO_i, taken over query rows ``chunk`` at a time
    (each row's O, LSE and D over all keys first)."""
    tau = 1.0 / np.sqrt(q.shape[1])
    out = {j: (np.zeros((block, k.shape[1])), np.zeros((block, v.shape[1]))) for j in blocks}
    for r0 in range(0, q.shape[0], chunk):
        qr, dor = q[r0:r0 + chunk], do[r0:r0 + chunk]
        o, lse = dense_rows(qr, k, v)
        dvec = (dor * o).sum(axis=1)
        for j in blocks:
            keys = slice(j * block, (j + 1) * block)
            p = np.exp(tau * (qr @ k[keys].T) - lse[:, None])
            ds = p * (dor @ v[keys].T - dvec[:, None])
            out[j][0][:] += tau * (ds.T @ qr)
            out[j][1][:] += p.T @ dor
    return out


def sparsity(k_per_head: Sequence[int], n_blocks: int) -> float:
    """Fraction of (head, group, block) attention tiles that the selection skips: 1 - sum_h k_h / (H NB)."""
    return 1.0 - float(sum(int(x) for x in k_per_head)) / (len(k_per_head) * n_blocks)


def use_sparse(k_per_head: Sequence[int], n_blocks: int, threshold: float) -> bool:
    """The dispatcher's rule: sparse attention iff the sparsity exceeds the threshold."""
    return sparsity(k_per_head, n_blocks) > threshold


# ----------------------------------------------------------------------------
# Stage 1: training the predictor (hi §2.A stage 1, nl §2.A fase 1: the
# low-rank predictors are trained for every head in parallel with the normal,
# full-attention training, through a loss that keeps the relative magnitude of
# the estimated scores)
# ----------------------------------------------------------------------------

def predictor_loss_head(q, k, wq, wk, group, block=BLOCK):
    """Loss of one (b, h).  With the predictor's block scores S = tau qhat khat^T and the true pooled
    logits T = tau qbar kbar^T (qbar, kbar the group and block means: T is the mean of tau Q K^T over each
    G x 64 tile), E = (S - T) minus each row's mean, and L = mean over the NG x NB entries of E^2.  Removing
    the row mean keeps only the relative magnitudes within a row, the part a softmax and a top-k see.
    Returns (L, E, qbar, kbar, qhat, khat)."""
    tau = 1.0 / np.sqrt(q.shape[1])
    qbar, kbar = pool_mean(q, group), pool_mean(k, block)
    qhat, khat = qbar @ wq, kbar @ wk
    diff = tau * (qhat @ khat.T) - tau * (qbar @ kbar.T)
    e = diff - diff.mean(axis=1, keepdims=True)
    return float((e * e).mean()), e, qbar, kbar, qhat, khat


def predictor_loss_grad_head(q, k, wq, wk, group, block=BLOCK):
    """(L, dL/dW_q, dL/dW_k) of one (b, h).  dL/dS = 2 E / (NG NB) (E already has zero row means, so the
    mean removal adds nothing), S = tau (qbar W_q)(kbar W_k)^T: dW_q = tau qbar^T dS khat,
    dW_k = tau kbar^T dS^T qhat."""
    tau = 1.0 / np.sqrt(q.shape[1])
    loss, e, qbar, kbar, qhat, khat = predictor_loss_head(q, k, wq, wk, group, block)
    ds = 2.0 * e / e.size
    return loss, tau * (qbar.T @ (ds @ khat)), tau * (kbar.T @ (ds.T @ qhat))


def predictor_loss_grad(q, k, wq, wk, group, block=BLOCK):
    """Per head h, averaged over the batch: loss [H], dW_q [H, d, r], dW_k [H, d, r] for inputs
    [B, H, N, d] and weights [H, d, r]."""
    B, H = q.shape[:2]
    loss = np.zeros(H)
    dwq, dwk = np.zeros(wq.shape), np.zeros(wk.shape)
    for h in range(H):
        for b in range(B):
            l, gq, gk = predictor_loss_grad_head(q[b, h], k[b, h], wq[h], wk[h], group, block)
            loss[h] += l / B
            dwq[h] += gq / B
            dwk[h] += gk / B
    return loss, dwq, dwk
