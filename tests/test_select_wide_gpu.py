"""Selection on wide rows and adversarial score distributions, against the oracle.

The selection kernels hold a row's NB scores in registers (up to 128 per lane at NB = 8,192) and find the
k-th largest through a first histogram level linear in score, then either an exact ranking of at most 64
candidates or further levels over the order-preserving keys of the bucket.  The cases reach each path at
the widest rows:
  - Gaussian scores (first level, then the exact ranking);
  - a handful of distinct values (buckets far above 64 keys, ties at the cut-off: the key-space levels);
  - magnitudes from 1e-30 to 1e30 with signed zeros, denormals and infinities (the first level's range is
    unusable: key space from the start);
  - constant rows (every score equal: the lowest ids win);
  - k = 1 and k = NB, and rows of 1,100 to 8,192 blocks (16 to 128 scores per lane);
  - the streamed selection at NB = 8,192 (scores computed in-kernel, dumped for the check);
  - coverage selection on wide rows.
The oracle's top-k of the same fp32 scores must equal the GPU's ids bit for bit, and the reverse index
must equal the oracle's.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import dynamic_sparse_attention_qk_amd as dsa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


def _scores(kind: str, ng: int, nb: int, rng: np.random.Generator) -> np.ndarray:
    if kind == "gauss":
        return rng.standard_normal((ng, nb)).astype(np.float32)
    if kind == "few":
        vals = np.array([-1.5, 0.0, 0.25, np.nextafter(np.float32(0.25), np.float32(1)), 3.0], dtype=np.float32)
        return rng.choice(vals, size=(ng, nb)).astype(np.float32)
    if kind == "range":
        mag = 10.0 ** rng.uniform(-30, 30, size=(ng, nb))
        s = (np.where(rng.random((ng, nb)) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
        u = rng.random((ng, nb))
        s[u < 0.02] = np.float32(0.0)
        s[(u >= 0.02) & (u < 0.03)] = np.float32(-0.0)
        s[(u >= 0.03) & (u < 0.04)] = np.float32(1e-40)        # a denormal
        s[(u >= 0.04) & (u < 0.045)] = np.float32(np.inf)
        s[(u >= 0.045) & (u < 0.05)] = np.float32(-np.inf)
        return s
    if kind == "const":
        s = np.full((ng, nb), 0.7, dtype=np.float32)
        s[1::2] = np.float32(0.0)
        s[1::2, ::3] = np.float32(-0.0)                          # rows of signed zeros: all equal
        return s
    raise ValueError(kind)


def _select(scores: np.ndarray, kph, group: int, coverage=None):
    """Materialised selection of scores [H, NG, NB] (B = 1) through the binding."""
    H, NG, NB = scores.shape
    p = dsa.Problem(batch=1, heads=H, seq_len=NB * 64, head_dim=64, rank=16, group=group)
    assert p.n_groups == NG
    plan = dsa.SparseAttentionPlan(p, kph, backward=False, coverage=coverage)
    plan.scores.copy_(torch.from_numpy(scores[None]))
    plan.idx.fill_(-7)
    plan.select()
    torch.cuda.synchronize()
    return plan


def _check_lists(plan, h: int, rows: np.ndarray):
    """Reverse index of head h (B = 1) equal to the oracle's of the kept rows."""
    p = plan.p
    base = int(plan.row_base[h])
    rp = plan.rev_ptr.cpu().numpy()[h]
    ptr, groups = oracle.reverse_index_csr(rows, p.n_blocks)
    assert np.array_equal(rp, ptr), f"rev_ptr of head {h}"
    got = plan.rev_idx.cpu().numpy()[base: base + int(ptr[-1])]
    assert np.array_equal(got, groups), f"rev_idx of head {h}"


CASES = [  # name, NB, G, k per head, kind
    ("gauss_8192", 8192, 128, [1904], "gauss"),
    ("few_values_4100", 4100, 128, [1, 777], "few"),
    ("range_2100", 2100, 128, [5, 2100], "range"),
    ("const_1500", 1500, 128, [1, 1499], "const"),
    ("gauss_1100_knb", 1100, 64, [1100, 3], "gauss"),
]


@pytest.mark.parametrize("name,nb,group,kph,kind", CASES, ids=[c[0] for c in CASES])
def test_wide_topk(name, nb, group, kph, kind):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    ng = nb * 64 // group
    scores = np.stack([_scores(kind, ng, nb, rng) for _ in kph])
    print(f"CASE {name} NB={nb} NG={ng} k={kph}", flush=True)
    plan = _select(scores, kph, group)
    idx = plan.idx.cpu().numpy()
    for h, k in enumerate(kph):
        base = int(plan.row_base[h])
        rows = idx[base: base + ng * k].reshape(ng, k)
        want = oracle.select_rows(scores[h].astype(np.float64), k)
        bad = np.nonzero(~np.all(rows == want, axis=1))[0]
        assert bad.size == 0, f"head {h}: {bad.size} rows differ, first {bad[:5]}"
        _check_lists(plan, h, rows)


def test_wide_streamed_matches_its_scores():
    """Streamed selection at NB = 8,192 (r = 32): the ids are the oracle's top-k of the scores the kernel
    computed (dumped), which match float64 dot products to the row-relative bound."""
    nb, group, k = 8192, 128, 1500
    ng = nb * 64 // group
    rng = np.random.default_rng(77)
    p = dsa.Problem(batch=1, heads=1, seq_len=nb * 64, head_dim=128, rank=32, group=group)
    plan = dsa.SparseAttentionPlan(p, [k], materialise_scores=False, backward=False)
    qh = rng.standard_normal((ng, 32)).astype(np.float32)
    kh = rng.standard_normal((nb, 32)).astype(np.float32)
    plan.qhat.copy_(torch.from_numpy(qh).view(1, 1, ng, 32))
    plan.khat.copy_(torch.from_numpy(kh).view(1, 1, nb, 32))
    dump = torch.empty(1, 1, ng, nb, dtype=torch.float32, device="cuda")
    plan.select(scores_dump=dump)
    torch.cuda.synchronize()
    s = dump.cpu().numpy()[0, 0]
    ref = (qh.astype(np.float64) @ kh.astype(np.float64).T) / np.sqrt(128.0)
    err = np.max(np.abs(s - ref), axis=1) / np.max(np.abs(ref), axis=1)
    assert err.max() <= 1e-3, err.max()
    rows = plan.idx.cpu().numpy()[: ng * k].reshape(ng, k)
    want = oracle.select_rows(s.astype(np.float64), k)
    bad = np.nonzero(~np.all(rows == want, axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"
    _check_lists(plan, 0, rows)


def test_wide_coverage():
    """Coverage selection (0.9 of the estimated mass, cap NB / 3) on 4,100-block rows: every count valid
    (the float64 top-c mass reaches the target, top-(c-1) does not, both to 1e-4), the ids the top-c."""
    nb, group, cov = 4100, 128, 0.9
    ng = nb * 64 // group
    cap = nb // 3
    rng = np.random.default_rng(78)
    scores = (3.0 * rng.standard_normal((1, ng, nb))).astype(np.float32)
    scores[0, ::7] = np.float32(0.5)   # flat rows: the cap binds
    plan = _select(scores, [cap], group, coverage=cov)
    idx = plan.idx.cpu().numpy()[: ng * cap].reshape(ng, cap)
    cnt = plan.cnt.cpu().numpy()[0, 0]
    for g in range(ng):
        s = scores[0, g].astype(np.float64)
        c = int(cnt[g])
        assert 1 <= c <= cap, (g, c)
        assert np.array_equal(idx[g, :c], oracle.select_row(s, c)), g
        assert (idx[g, c:] == -1).all(), g
        want = len(oracle.select_coverage_row(s, cov, cap))
        if c != want:  # allowed only where fp32 and float64 sums straddle the target
            order = np.lexsort((np.arange(nb), -s))
            cum = np.cumsum(oracle.block_mass(s)[order])
            assert cum[c - 1] >= cov - 1e-4 and (c == 1 or cum[c - 2] <= cov + 1e-4), (g, c, want)
