"""Pins of the float64 oracle against things other than itself (CPU only).

Each check is a function raising AssertionError; the mutation tests at the end
plant plausible mistakes into the oracle (on the CPU) and confirm that at least
one pin fails for each.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import dsv_oracle as O
from tests import brute
import synth


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _tiny(seed=0, n=256, d=16, r=8, clustered=True):
    rng = _rng(seed)
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    if clustered:   # give the selection real structure: a few shared directions
        cent = rng.standard_normal((4, d)) * 2.0
        lab = rng.integers(0, 4, size=n)
        q += cent[lab]
        k += cent[lab]
    v = rng.standard_normal((n, d))
    do = rng.standard_normal((n, d))
    wq = rng.standard_normal((d, r)) / math.sqrt(d)
    wk = rng.standard_normal((d, r)) / math.sqrt(d)
    return q, k, v, do, wq, wk


# ---------------------------------------------------------------------------- checks

def check_scores_brute(seed=1, group=64, n=256, d=16, r=8):
    q, k, _, _, wq, wk = _tiny(seed, n=n, d=d, r=r)
    qhat, khat, s = O.predict_head(q, k, wq, wk, group)
    ref = brute.tile_mean_scores(q, k, wq, wk, group)
    assert qhat.shape == (n // group, r) and khat.shape == (n // 64, r)
    np.testing.assert_allclose(s, ref, rtol=1e-11, atol=1e-12)


def check_identity_predictor(seed=2, group=64):
    q, k, _, _, _, _ = _tiny(seed, n=384, d=16)
    eye = np.eye(16)
    _, _, s = O.predict_head(q, k, eye, eye, group)
    ref = brute.true_tile_mean(q, k, group)
    np.testing.assert_allclose(s, ref, rtol=1e-11, atol=1e-12)
    for kk in (1, 2, 6):
        for g in range(s.shape[0]):
            assert list(O.select_row(s[g], kk)) == brute.topk_sorted(ref[g], kk)


def check_select_brute(seed=3):
    rng = _rng(seed)
    for trial in range(60):
        nb = int(rng.integers(1, 70))
        vals = np.array([0.0, -0.0, 1.5, -2.0, 3.25, 1e-30, -1e-30, 7.0])
        row = rng.choice(vals, size=nb) if trial % 2 else rng.standard_normal(nb)
        for kk in {1, nb, int(rng.integers(1, nb + 1))}:
            assert list(O.select_row(row, kk)) == brute.topk_sorted(row, kk), (row, kk)


def check_select_special():
    row = np.array([0.5, 2.0, 2.0, -1.0, 2.0])
    assert list(O.select_row(row, 1)) == [1]                 # argmax, lowest id among equals
    assert list(O.select_row(row, 2)) == [1, 2]
    assert list(O.select_row(row, 5)) == [0, 1, 2, 3, 4]     # k = NB keeps all
    row0 = np.array([-0.0, 0.0, -3.0])
    assert list(O.select_row(row0, 1)) == [0]                # -0.0 == +0.0: lowest id
    row1 = np.array([-1.0, 0.0, -0.0])
    assert list(O.select_row(row1, 1)) == [1]


def check_select_rows_vectorised(seed=31):
    # the whole-matrix selection equals the Python sort row by row: heavy ties, +-0.0, tiny values, k = 1, NB
    rng = _rng(seed)
    vals = np.array([0.0, -0.0, 1.5, -2.0, 3.25, 1e-30, -1e-30, 7.0])
    for trial in range(12):
        ng, nb = int(rng.integers(1, 20)), int(rng.integers(1, 90))
        s = rng.choice(vals, size=(ng, nb)) if trial % 2 else rng.standard_normal((ng, nb))
        for kk in {1, nb, int(rng.integers(1, nb + 1))}:
            got = O.select_rows(s, kk)
            assert got.shape == (ng, kk)
            for g in range(ng):
                assert list(got[g]) == brute.topk_sorted(s[g], kk), (trial, g, kk)


def check_duplicate_blocks_tie():
    q, k, _, _, wq, wk = _tiny(4, n=512, d=16)
    # blocks 1, 4 and 6 are bitwise copies of block 6's keys: their scores are equal
    for j in (1, 4):
        k[j * 64:(j + 1) * 64] = k[6 * 64:7 * 64]
    _, _, s = O.predict_head(q, k, wq, wk, 64)
    for g in range(s.shape[0]):
        assert s[g, 1] == s[g, 4] == s[g, 6]
        order = brute.topk_sorted(s[g], 8)
        for kk in range(1, 9):
            sel = list(O.select_row(s[g], kk))
            assert sel == brute.topk_sorted(s[g], kk)
            chosen_dup = [j for j in (1, 4, 6) if j in sel]
            assert chosen_dup == [1, 4, 6][:len(chosen_dup)]   # lowest ids win the tie
        assert order == list(range(8))


def check_linearity(seed=5):
    q, k, _, _, wq, wk = _tiny(seed)
    _, _, s = O.predict_head(q, k, wq, wk, 64)
    _, _, s2 = O.predict_head(q, k, 3.0 * wq, wk, 64)
    np.testing.assert_allclose(s2, 3.0 * s, rtol=1e-12, atol=1e-13)
    for g in range(s.shape[0]):
        assert (O.select_row(s[g], 2) == O.select_row(s2[g], 2)).all()


def _sel(s, kk):
    return np.stack([O.select_row(s[g], kk) for g in range(s.shape[0])])


def check_forward_brute(seed=6, group=64, kk=2, n=256):
    q, k, v, _, wq, wk = _tiny(seed, n=n)
    _, _, s = O.predict_head(q, k, wq, wk, group)
    idx = _sel(s, kk)
    o, lse = O.forward_head(q, k, v, idx, group)
    mask = brute.mask_from_idx(idx, n, group)
    o_ref, lse_ref, p_ref = brute.masked_attention(q, k, v, mask)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
    # rows of P sum to one; V = 1 gives O = 1; one-hot V (V = I) exposes P itself
    for g in range(n // group):
        rows = slice(g * group, (g + 1) * group)
        keys = O.kept_keys(idx[g])
        _, _, p = O.group_forward(q[rows], k, v, keys)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        ones, _, _ = O.group_forward(q[rows], k, np.ones_like(v), keys)
        np.testing.assert_allclose(ones, 1.0, rtol=0, atol=1e-12)
        eye_o, _, _ = O.group_forward(q[rows], k, np.eye(n), keys)
        np.testing.assert_allclose(eye_o, p_ref[rows], rtol=1e-11, atol=1e-13)


def check_dense_equals_sdpa(seed=7, n=256, d=16):
    q, k, v, do, _, _ = _tiny(seed, n=n, d=d)
    nb = n // 64
    idx = np.tile(np.arange(nb), (n // 64, 1))               # k = NB: every block kept
    o, lse = O.forward_head(q, k, v, idx, 64)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    np.testing.assert_allclose(o, ref.detach().numpy(), rtol=1e-11, atol=1e-12)
    lse_ref = torch.logsumexp(tq @ tk.T / math.sqrt(d), dim=1)
    np.testing.assert_allclose(lse, lse_ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    (ref * torch.tensor(do)).sum().backward()
    dq, dk, dv = O.backward_head(q, k, v, do, idx, 64)
    for mine, theirs in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, theirs.grad.numpy(), rtol=1e-10, atol=1e-11)


def check_sparse_equals_masked_sdpa(seed=8, group=128, n=512, kk=3):
    q, k, v, do, wq, wk = _tiny(seed, n=n)
    _, _, s = O.predict_head(q, k, wq, wk, group)
    idx = _sel(s, kk)
    mask = torch.tensor(brute.mask_from_idx(idx, n, group))
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mask[None])[0]
    o, _ = O.forward_head(q, k, v, idx, group)
    np.testing.assert_allclose(o, ref.detach().numpy(), rtol=1e-11, atol=1e-12)
    (ref * torch.tensor(do)).sum().backward()
    dq, dk, dv = O.backward_head(q, k, v, do, idx, group)
    for mine, theirs in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, theirs.grad.numpy(), rtol=1e-10, atol=1e-11)


def check_finite_differences(seed=9):
    n, d = 128, 4
    q, k, v, do, wq, wk = _tiny(seed, n=n, d=d, r=2)
    idx = np.array([[1], [0]])                               # group 0 sees block 1, group 1 sees block 0
    dq, dk, dv = O.backward_head(q, k, v, do, idx, 64)
    fq, fk, fv = brute.finite_diff_grads(q, k, v, do, brute.mask_from_idx(idx, n, 64))
    for mine, fd in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(mine, fd, rtol=1e-6, atol=1e-7)


def check_gradient_invariants(seed=10, n=512, kk=2):
    q, k, v, do, wq, wk = _tiny(seed, n=n)
    _, _, s = O.predict_head(q, k, wq, wk, 64)
    idx = _sel(s, kk)
    dq, dk, dv = O.backward_head(q, k, v, do, idx, 64)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-10)            # rows of dS sum to 0
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-10)  # rows of P sum to 1
    kept = np.zeros(n // 64, dtype=bool)
    kept[np.unique(idx)] = True
    for j in np.nonzero(~kept)[0]:
        assert (dk[j * 64:(j + 1) * 64] == 0).all() and (dv[j * 64:(j + 1) * 64] == 0).all()


def check_sampled_match_full(seed=11, n=768, group=64, kk=3):
    q, k, v, do, wq, wk = _tiny(seed, n=n)
    _, _, s = O.predict_head(q, k, wq, wk, group)
    idx = _sel(s, kk)
    o, lse = O.forward_head(q, k, v, idx, group)
    o2, lse2 = O.forward_head(q, k, v, idx, group, groups=[0, 5])
    np.testing.assert_array_equal(o2[:64], o[:64])
    np.testing.assert_array_equal(lse2[5 * 64:6 * 64], lse[5 * 64:6 * 64])
    assert np.isnan(o2[64:128]).all()
    dq, dk, dv = O.backward_head(q, k, v, do, idx, group)
    for g, rows in O.dq_groups(q, k, v, do, idx, group, [1, 7]).items():
        np.testing.assert_allclose(rows, dq[g * 64:(g + 1) * 64], rtol=1e-12, atol=1e-13)
    for j, (dkj, dvj) in O.dkdv_blocks(q, k, v, do, idx, group, [0, 3, 11]).items():
        np.testing.assert_allclose(dkj, dk[j * 64:(j + 1) * 64], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dvj, dv[j * 64:(j + 1) * 64], rtol=1e-11, atol=1e-12)


def check_reverse_index(seed=12):
    rng = _rng(seed)
    nb, ng, kk = 13, 9, 4
    idx = np.stack([np.sort(rng.choice(nb, kk, replace=False)) for _ in range(ng)])
    rev = O.reverse_index(idx, nb)
    for j in range(nb):
        assert list(rev[j]) == [g for g in range(ng) if j in set(idx[g])]
        assert list(O.reverse_list(idx, j)) == list(rev[j])


def check_reverse_index_csr(seed=32):
    # the compressed reverse index equals a membership scan block by block, on ragged random lists
    rng = _rng(seed)
    for nb, ng, kk in ((13, 9, 4), (40, 25, 1), (7, 30, 7), (64, 3, 20)):
        idx = np.stack([np.sort(rng.choice(nb, kk, replace=False)) for _ in range(ng)])
        ptr, groups = O.reverse_index_csr(idx, nb)
        assert ptr[0] == 0 and ptr[-1] == idx.size and (np.diff(ptr) >= 0).all()
        for j in range(nb):
            assert list(groups[ptr[j]:ptr[j + 1]]) == [g for g in range(ng) if j in set(idx[g].tolist())]


def check_dkdv_block_part(seed=33, n=768, group=64, kk=4):
    # the per-group parts of a block, summed over its reverse list, equal the full backward's dK, dV rows
    q, k, v, do, wq, wk = _tiny(seed, n=n)
    _, _, s = O.predict_head(q, k, wq, wk, group)
    idx = _sel(s, kk)
    _, dk, dv = O.backward_head(q, k, v, do, idx, group)
    ptr, groups = O.reverse_index_csr(idx, n // 64)
    for j in range(n // 64):
        gk, gv = np.zeros((64, 16)), np.zeros((64, 16))
        for g in groups[ptr[j]:ptr[j + 1]]:
            pk, pv = O.dkdv_block_part(q, k, v, do, idx[g], group, int(g), j)
            gk += pk
            gv += pv
        np.testing.assert_allclose(gk, dk[j * 64:(j + 1) * 64], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(gv, dv[j * 64:(j + 1) * 64], rtol=1e-11, atol=1e-12)


def check_batched_api(seed=13):
    w = synth.workload(1).with_(grid=(2, 8, 16), heads=2, k=2)
    inp = synth.generate(w)
    q, k, v = inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v")
    wt = inp.w.astype(np.float64)
    qhat, khat, s = O.predict(q, k, wt, wt, w.group)
    idx = O.select(s, inp.k_per_head)
    o, lse = O.forward(q, k, v, idx, w.group)
    for h in range(2):
        _, _, sh = O.predict_head(q[0, h], k[0, h], wt[h], wt[h], w.group)
        np.testing.assert_array_equal(s[0, h], sh)
        mask = brute.mask_from_idx(idx[0][h], w.seq_len, w.group)
        o_ref, lse_ref, _ = brute.masked_attention(q[0, h], k[0, h], v[0, h], mask)
        np.testing.assert_allclose(o[0, h], o_ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], lse_ref, rtol=1e-12, atol=1e-12)


def _tiny_selection(seed, n=512, d=16, r=8, group=64, kk=5):
    q, k, v, do, wq, wk = _tiny(seed, n=n, d=d, r=r)
    _, _, s = O.predict_head(q, k, wq, wk, group)
    idx = np.stack([O.select_row(s[g], kk) for g in range(n // group)])
    return q, k, v, idx


def check_split_bounds():
    for k in (1, 2, 5, 13, 90):
        for n in (1, 2, 3, 4, 7, 16, 100):
            b = O.split_bounds(k, n)
            assert len(b) == n and b[0][0] == 0 and b[-1][1] == k
            assert all(b[i][1] == b[i + 1][0] for i in range(n - 1))   # contiguous
            sizes = [e - a for a, e in b]
            assert max(sizes) - min(sizes) <= 1 and sum(sizes) == k


def check_split_merge_equals_unsplit(seed=31, group=64, kk=5):
    """Any partition of the kept lists, merged, is the unsplit attention (brute-force masked softmax)."""
    q, k, v, idx = _tiny_selection(seed, group=group, kk=kk)
    n = q.shape[0]
    o_ref, lse_ref, _ = brute.masked_attention(q, k, v, brute.mask_from_idx(idx, n, group))
    for n_split in (1, 2, 3, kk, kk + 3):     # kk + 3 leaves some parts empty
        o_p, lse_p = O.forward_split_head(q, k, v, idx, group, n_split)
        o, lse = O.merge_states(list(o_p), list(lse_p))
        np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def check_partial_states_brute(seed=32, group=64, kk=5, n_split=3):
    """Each part's state is the masked softmax over that part's blocks alone."""
    q, k, v, idx = _tiny_selection(seed, group=group, kk=kk)
    n = q.shape[0]
    o_p, lse_p = O.forward_split_head(q, k, v, idx, group, n_split)
    for s, (a, e) in enumerate(O.split_bounds(kk, n_split)):
        mask = brute.mask_from_idx(idx[:, a:e], n, group)
        o_ref, lse_ref, _ = brute.masked_attention(q, k, v, mask)
        np.testing.assert_allclose(o_p[s], o_ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse_p[s], lse_ref, rtol=1e-12, atol=1e-12)
    # an empty part: O = 0, LSE = -inf
    o_e, lse_e = O.partial_state(q[:group], k, v, np.zeros(0, dtype=np.int64))
    assert (o_e == 0).all() and np.isneginf(lse_e).all()


def check_merge_algebra(seed=33):
    """Associative, commutative, identity on one part, and a -inf part contributes nothing."""
    rng = _rng(seed)
    parts = [(rng.standard_normal((7, 5)), rng.standard_normal(7) * 3.0) for _ in range(4)]
    os_, ls_ = [p[0] for p in parts], [p[1] for p in parts]
    o_all, l_all = O.merge_states(os_, ls_)
    o12, l12 = O.merge_states(os_[:2], ls_[:2])
    o34, l34 = O.merge_states(os_[2:], ls_[2:])
    o_t, l_t = O.merge_states([o12, o34], [l12, l34])
    np.testing.assert_allclose(o_t, o_all, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l_t, l_all, rtol=1e-13, atol=1e-13)
    perm = [2, 0, 3, 1]
    o_p, l_p = O.merge_states([os_[i] for i in perm], [ls_[i] for i in perm])
    np.testing.assert_allclose(o_p, o_all, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l_p, l_all, rtol=1e-13, atol=1e-13)
    o1, l1 = O.merge_states(os_[:1], ls_[:1])
    np.testing.assert_allclose(o1, os_[0], rtol=1e-15, atol=0)
    np.testing.assert_allclose(l1, ls_[0], rtol=1e-15, atol=0)
    o_n, l_n = O.merge_states(os_[:2] + [np.full((7, 5), 9.0)], ls_[:2] + [np.full(7, -np.inf)])
    np.testing.assert_allclose(o_n, o12, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l_n, l12, rtol=1e-14, atol=1e-14)
    # closed form for two parts with equal LSE: the plain mean of the outputs, LSE + ln 2
    o_eq, l_eq = O.merge_states([os_[0], os_[1]], [ls_[0], ls_[0]])
    np.testing.assert_allclose(o_eq, 0.5 * (os_[0] + os_[1]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l_eq, ls_[0] + math.log(2.0), rtol=1e-14, atol=1e-14)


def check_dense_sdpa(seed=31, n=320, d=16):
    # full attention against torch's scaled_dot_product_attention and autograd in float64
    q, k, v, do, _, _ = _tiny(seed, n=n, d=d)
    o, lse = O.dense_forward_head(q, k, v)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    np.testing.assert_allclose(o, ref.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(tq @ tk.T / math.sqrt(d), dim=1).detach().numpy(),
                               rtol=1e-12, atol=1e-12)
    (ref * torch.tensor(do)).sum().backward()
    for mine, theirs in zip(O.dense_backward_head(q, k, v, do), (tq, tk, tv)):
        np.testing.assert_allclose(mine, theirs.grad.numpy(), rtol=1e-10, atol=1e-11)


def check_dense_brute(seed=32, n=64, d=4):
    # an all-true mask in the brute-force attention, and central differences of sum(dO * O)
    q, k, v, do, _, _ = _tiny(seed, n=n, d=d, r=2)
    mask = np.ones((n, n), dtype=bool)
    o_ref, lse_ref, _ = brute.masked_attention(q, k, v, mask)
    o, lse = O.dense_forward_head(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
    for mine, fd in zip(O.dense_backward_head(q, k, v, do), brute.finite_diff_grads(q, k, v, do, mask)):
        np.testing.assert_allclose(mine, fd, rtol=1e-5, atol=1e-7)


def check_dense_closed_forms(seed=33, n=192, d=8):
    q, _, v, do, _, _ = _tiny(seed, n=n, d=d)
    k0 = np.zeros((n, d))                                       # equal logits: uniform attention
    o, lse = O.dense_forward_head(q, k0, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(n), rtol=1e-14, atol=1e-14)
    _, _, dv = O.dense_backward_head(q, k0, v, do)
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=0), dv.shape), rtol=1e-12, atol=1e-13)
    # any inputs: rows of P sum to 1, so the dV rows add up to the dO rows; dS rows sum to 0, so dK sums to 0
    q, k, v, do, _, _ = _tiny(seed + 1, n=n, d=d)
    _, dk, dv = O.dense_backward_head(q, k, v, do)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    # a key that is a copy of another gets the same gradient rows
    k2 = k.copy()
    k2[5] = k2[70]
    _, dk2, dv2 = O.dense_backward_head(q, k2, np.where(np.arange(n)[:, None] == 5, v[70], v), do)
    np.testing.assert_allclose(dk2[5], dk2[70], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv2[5], dv2[70], rtol=1e-11, atol=1e-12)


def check_dense_sampled(seed=34, n=448, d=8):
    # the row- and block-sampled evaluators against the full gradient (chunk 96: a ragged last chunk)
    q, k, v, do, _, _ = _tiny(seed, n=n, d=d)
    dq, dk, dv = O.dense_backward_head(q, k, v, do)
    rows = np.array([0, 1, 63, 64, 200, n - 1])
    np.testing.assert_allclose(O.dense_dq_rows(q, k, v, do, rows), dq[rows], rtol=1e-12, atol=1e-13)
    got = O.dense_dkdv_blocks(q, k, v, do, [0, 3, n // 64 - 1], chunk=96)
    for j, (a, b) in got.items():
        np.testing.assert_allclose(a, dk[j * 64:(j + 1) * 64], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(b, dv[j * 64:(j + 1) * 64], rtol=1e-11, atol=1e-12)
    o, lse = O.dense_forward_head(q, k, v)
    o_r, lse_r = O.dense_rows(q[rows], k, v)
    np.testing.assert_allclose(o_r, o[rows], rtol=1e-12, atol=1e-14)   # BLAS blocking varies with the row count
    np.testing.assert_allclose(lse_r, lse[rows], rtol=1e-14, atol=0)


def check_dispatch_rule():
    assert O.sparsity([16, 16], 16) == 0.0
    assert abs(O.sparsity([1, 3], 10) - 0.8) < 1e-15
    assert abs(O.sparsity([90] * 24, 900) - 0.9) < 1e-15
    assert not O.use_sparse([16, 16], 16, 0.0)          # nothing skipped: dense even at threshold 0
    assert not O.use_sparse([8, 8], 16, 0.5)            # exactly at the threshold: dense
    assert O.use_sparse([7, 8], 16, 0.5)
    assert O.use_sparse([1], 2, 0.0) and not O.use_sparse([1], 2, 0.5)


def _brute_pred_loss(q, k, wq, wk, group):
    # from the full N x N predicted and true logit matrices, averaged per tile (tests/brute.py)
    diff = brute.tile_mean_scores(q, k, wq, wk, group) - brute.true_tile_mean(q, k, group)
    e = diff - diff.mean(axis=1, keepdims=True)
    return float((e * e).mean())


def check_pred_loss_brute(seed=41, n=256, d=8, r=4, group=64):
    q, k, _, _, wq, wk = _tiny(seed, n=n, d=d, r=r)
    loss, gq, gk = O.predictor_loss_grad_head(q, k, wq, wk, group)
    assert abs(loss - _brute_pred_loss(q, k, wq, wk, group)) <= 1e-12 * max(1.0, loss)
    # central differences of the brute-force loss, entry by entry
    h = 1e-6
    for w, g, which in ((wq, gq, 0), (wk, gk, 1)):
        fd = np.zeros_like(w)
        for ix in np.ndindex(*w.shape):
            wp, wm = w.copy(), w.copy()
            wp[ix] += h
            wm[ix] -= h
            args_p = (wp, wk) if which == 0 else (wq, wp)
            args_m = (wm, wk) if which == 0 else (wq, wm)
            fd[ix] = (_brute_pred_loss(q, k, *args_p, group) - _brute_pred_loss(q, k, *args_m, group)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-5, atol=1e-9)


def check_pred_loss_closed_forms(seed=42, n=384, d=8, group=128):
    q, k, _, _, _, _ = _tiny(seed, n=n, d=d, r=d)
    eye = np.eye(d)
    loss, gq, gk = O.predictor_loss_grad_head(q, k, eye, eye, group)   # full-rank identity: S = T
    assert loss < 1e-28 and np.abs(gq).max() < 1e-14 and np.abs(gk).max() < 1e-14
    # a zero predictor: L is the mean square of the row-centred true pooled logits
    z = np.zeros((d, 3))
    t = brute.true_tile_mean(q, k, group)
    tc = t - t.mean(axis=1, keepdims=True)
    loss0, _, _ = O.predictor_loss_grad_head(q, k, z, z, group)
    assert abs(loss0 - float((tc * tc).mean())) <= 1e-12 * loss0
    # shifting every key by one vector moves each row of S and T by a constant: L is unchanged
    rng = _rng(seed)
    wq, wk = rng.standard_normal((d, 3)), rng.standard_normal((d, 3))
    c = rng.standard_normal(d) * 3.0
    l1, g1q, g1k = O.predictor_loss_grad_head(q, k, wq, wk, group)
    l2, g2q, _ = O.predictor_loss_grad_head(q, k + c, wq, wk, group)
    assert abs(l1 - l2) <= 1e-11 * l1
    np.testing.assert_allclose(g2q, g1q, rtol=1e-9, atol=1e-12)
    # batched form: the mean over the batch of the per-(b, h) values
    qb, kb = np.stack([q, q[::-1]])[:, None], np.stack([k, k[::-1]])[:, None]
    lb, gbq, gbk = O.predictor_loss_grad(qb, kb, wq[None], wk[None], group)
    l_r, gq_r, gk_r = O.predictor_loss_grad_head(q[::-1], k[::-1], wq, wk, group)
    np.testing.assert_allclose(lb[0], 0.5 * (l1 + l_r), rtol=1e-13)
    np.testing.assert_allclose(gbq[0], 0.5 * (g1q + gq_r), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(gbk[0], 0.5 * (g1k + gk_r), rtol=1e-12, atol=1e-15)


def _brute_coverage(row, coverage, cap):
    # Python sort of (-s, j) tuples, masses from math.exp normalised with math.fsum, accumulate to the target
    mx = max(float(x) for x in row)
    w = [math.exp(float(x) - mx) for x in row]
    z = math.fsum(w)
    pairs = sorted((-float(x), j) for j, x in enumerate(row))
    taken, acc = [], []
    for _, j in pairs:
        taken.append(j)
        acc.append(w[j] / z)
        if math.fsum(acc) >= coverage or len(taken) == cap:
            break
    return sorted(taken)


def check_coverage_brute(seed=51):
    rng = _rng(seed)
    for trial in range(60):
        nb = int(rng.integers(1, 40))
        row = rng.standard_normal(nb) * float(rng.choice([0.3, 1.0, 4.0]))
        if trial % 3 == 0:                                   # heavy ties
            row = np.round(row * 2) / 2
        for cov in (0.05, 0.5, 0.9, 0.99):
            for cap in (1, max(1, nb // 2), nb):
                got = list(O.select_coverage_row(row, cov, cap))
                want = _brute_coverage(row, cov, cap)
                if got != want:
                    # only a cumulative mass within rounding of the target may flip the count by one
                    m = np.sort(O.block_mass(row))[::-1]
                    c = min(len(got), len(want))
                    assert abs(len(got) - len(want)) == 1 and abs(m[:c].sum() - cov) < 1e-12, (row, cov, cap)
                else:
                    # a coverage selection is the top-c selection for its own c
                    assert got == list(O.select_row(row, len(got)))


def check_coverage_closed_forms():
    flat = np.zeros(16)
    for cov, c in ((0.5, 8), (0.25, 4), (1.0 / 16, 1), (0.9, 15), (1.0, 16)):
        assert list(O.select_coverage_row(flat, cov, 16)) == list(range(c)), cov   # uniform: ceil(cov NB), lowest ids
    peak = np.zeros(10)
    peak[7] = 50.0
    assert list(O.select_coverage_row(peak, 0.999, 10)) == [7]
    row = _rng(52).standard_normal(12)
    assert len(O.select_coverage_row(row, 1.0, 12)) == 12
    assert list(O.select_coverage_row(row, 0.999999, 3)) == list(O.select_row(row, 3))   # the cap
    np.testing.assert_allclose(O.block_mass(row).sum(), 1.0, rtol=1e-15)
    np.testing.assert_allclose(O.block_mass(row + 100.0), O.block_mass(row), rtol=1e-13)  # shift-invariant


def check_ragged_attention_brute(seed=53, n=384, group=64):
    # rows of different lengths: forward and backward against masked brute force and autograd
    q, k, v, do, _, _ = _tiny(seed, n=n, d=8)
    rng = _rng(seed)
    nb = n // 64
    idx = [np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False)) for _ in range(n // group)]
    mask = brute.mask_from_idx(idx, n, group)
    o_ref, lse_ref, _ = brute.masked_attention(q, k, v, mask)
    o, lse = O.forward_head(q, k, v, idx, group)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                           attn_mask=torch.tensor(mask)[None])[0]
    (ref * torch.tensor(do)).sum().backward()
    for mine, theirs in zip(O.backward_head(q, k, v, do, idx, group), (tq, tk, tv)):
        np.testing.assert_allclose(mine, theirs.grad.numpy(), rtol=1e-10, atol=1e-11)
    rev = O.reverse_index(idx, nb)
    for j in range(nb):
        assert list(rev[j]) == [g for g in range(len(idx)) if j in set(idx[g].tolist())]


def check_diagonal_brute(seed=54):
    rng = _rng(seed)
    for trial in range(40):
        group = int(rng.choice([64, 128]))
        ng = int(rng.integers(1, 9))
        nb = ng * group // 64
        g = int(rng.integers(0, ng))
        row = rng.standard_normal(nb) * float(rng.choice([0.5, 3.0]))
        if trial % 2:
            row = np.round(row)                            # ties
        own = list(range(g * group // 64, (g + 1) * group // 64))
        rest = [j for _, j in sorted((-float(row[j]), j) for j in range(nb) if j not in own)]
        for k in range(len(own), nb + 1):
            assert list(O.select_row_diag(row, k, g, group)) == sorted(own + rest[:k - len(own)])
        mx = max(float(x) for x in row)
        w = [math.exp(float(x) - mx) for x in row]
        z = math.fsum(w)
        for cov in (0.01, 0.5, 0.9, 1.0):
            for cap in (len(own), nb):
                taken = []
                for j in own + rest:
                    taken.append(j)
                    done = len(taken) >= len(own) and math.fsum(w[t] / z for t in taken) >= cov
                    if done or len(taken) == cap:
                        break
                got = list(O.select_coverage_row_diag(row, cov, cap, g, group))
                if got != sorted(taken):   # only a prefix mass within rounding of the target may differ
                    cum = np.cumsum(O.block_mass(row)[O.select_order(row, own)])
                    c = min(len(got), len(taken))
                    assert abs(len(got) - len(taken)) == 1 and abs(cum[c - 1] - cov) < 1e-12
    # the forced blocks alone when k is their number; without a diagonal the rules are the plain ones
    row = np.arange(8.0)
    assert list(O.select_row_diag(row, 2, 0, 128)) == [0, 1]
    assert list(O.select_row_diag(row, 3, 0, 128)) == [0, 1, 7]
    assert list(O.select_order(row)) == list(range(7, -1, -1))


def check_pooled_scores_brute(seed=56, n=256, d=8, r=4, group=128):
    q, k, _, _, wq, wk = _tiny(seed, n=n, d=d, r=r)
    tau = 1.0 / math.sqrt(d)
    pq, pk = q @ wq, k @ wk
    ng, nb = n // group, n // 64
    for pooling in ("max", "lse", "mean"):
        got = O.predict_head_pooled(q, k, wq, wk, group, pooling)
        for g in range(ng):
            for j in range(nb):
                vals = [tau * float(pq[i] @ pk[m]) for i in range(g * group, (g + 1) * group)
                        for m in range(j * 64, (j + 1) * 64)]
                if pooling == "max":
                    want = max(vals)
                elif pooling == "mean":
                    want = math.fsum(vals) / len(vals)
                else:
                    mx = max(vals)
                    want = mx + math.log(math.fsum(math.exp(v - mx) for v in vals) / len(vals))
                assert abs(got[g, j] - want) <= 1e-12 * max(1.0, abs(want)), (pooling, g, j)
    # mean pooling of the token logits is the pooled-proxy score of predict_head
    np.testing.assert_allclose(O.predict_head_pooled(q, k, wq, wk, group, "mean"),
                               O.predict_head(q, k, wq, wk, group)[2], rtol=1e-11, atol=1e-12)
    # mean <= lse <= max, tile by tile; equal logits make all three equal
    mean, lse, mx = (O.predict_head_pooled(q, k, wq, wk, group, x) for x in ("mean", "lse", "max"))
    assert (mean <= lse + 1e-12).all() and (lse <= mx + 1e-12).all()
    z = np.zeros((d, r))
    for x in ("mean", "lse", "max"):
        np.testing.assert_allclose(O.predict_head_pooled(q, k, z, z, group, x), 0.0, atol=1e-15)
        # the row-sampled evaluator equals the full one
        full = O.predict_head_pooled(q, k, wq, wk, group, x)
        for g, row in O.predict_head_pooled_groups(q, k, wq, wk, group, x, [0, ng - 1]).items():
            np.testing.assert_allclose(row, full[g], rtol=1e-12, atol=1e-13)


ALL_CHECKS = [
    check_scores_brute, check_identity_predictor, check_select_brute, check_select_special,
    check_duplicate_blocks_tie, check_linearity, check_forward_brute, check_dense_equals_sdpa,
    check_sparse_equals_masked_sdpa, check_finite_differences, check_gradient_invariants,
    check_sampled_match_full, check_reverse_index, check_batched_api, check_split_bounds,
    check_split_merge_equals_unsplit, check_partial_states_brute, check_merge_algebra, check_dense_sdpa,
    check_dense_brute, check_dense_closed_forms, check_dense_sampled, check_dispatch_rule,
    check_pred_loss_brute, check_pred_loss_closed_forms, check_coverage_brute, check_coverage_closed_forms,
    check_ragged_attention_brute, check_diagonal_brute, check_pooled_scores_brute, check_select_rows_vectorised,
    check_reverse_index_csr, check_dkdv_block_part,
]


# ---------------------------------------------------------------------------- tests

@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_scores_group128():
    check_scores_brute(seed=21, group=128, n=512)


def test_forward_group128():
    check_forward_brute(seed=22, group=128, kk=3, n=512)


# ---------------------------------------------------------------------------- mutations

def _fails_some_pin(monkeypatch, target, replacement, checks):
    monkeypatch.setattr(O, target, replacement)
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    monkeypatch.undo()
    return failed


def test_mutation_pool_sum_instead_of_mean(monkeypatch):
    def bad(x, size):
        n, d = x.shape
        return x.reshape(n // size, size, d).sum(axis=1)
    assert _fails_some_pin(monkeypatch, "pool_mean", bad, [check_scores_brute, check_identity_predictor])


def test_mutation_scale_by_rank(monkeypatch):
    def bad(q, k, wq, wk, group, block=64):
        qhat = O.pool_mean(q, group) @ wq
        khat = O.pool_mean(k, block) @ wk
        return qhat, khat, (qhat @ khat.T) / math.sqrt(wq.shape[1])
    assert _fails_some_pin(monkeypatch, "predict_head", bad, [check_scores_brute])


def test_mutation_swapped_predictors(monkeypatch):
    orig = O.predict_head

    def bad(q, k, wq, wk, group, block=64):
        return orig(q, k, wk, wq, group, block)
    assert _fails_some_pin(monkeypatch, "predict_head", bad, [check_scores_brute])


def test_mutation_ties_to_highest_id(monkeypatch):
    def bad(row, k):
        nb = row.shape[0]
        order = np.lexsort((-np.arange(nb), -np.asarray(row)))
        return np.sort(order[:k])
    assert _fails_some_pin(monkeypatch, "select_row", bad, [check_select_brute, check_select_special,
                                                            check_duplicate_blocks_tie])


def test_mutation_select_smallest(monkeypatch):
    def bad(row, k):
        return np.sort(np.argsort(np.asarray(row), kind="stable")[:k])
    assert _fails_some_pin(monkeypatch, "select_row", bad, [check_select_brute, check_identity_predictor])


def test_mutation_kept_keys_off_by_block(monkeypatch):
    def bad(idx_row, block=64):
        return (np.asarray(idx_row)[:, None] * (block - 1) + np.arange(block)[None, :]).ravel()
    assert _fails_some_pin(monkeypatch, "kept_keys", bad, [check_forward_brute])


def test_mutation_no_scale_in_logits(monkeypatch):
    def bad(qg, k, v, keys):
        logits = qg @ k[keys].T
        m = logits.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(logits - m).sum(axis=1))
        p = np.exp(logits - lse[:, None])
        return p @ v[keys], lse, p
    assert _fails_some_pin(monkeypatch, "group_forward", bad, [check_forward_brute, check_dense_equals_sdpa])


def test_mutation_backward_missing_D(monkeypatch):
    def bad(qg, k, v, dog, keys):
        tau = 1.0 / np.sqrt(qg.shape[1])
        og, lse, p = O.group_forward(qg, k, v, keys)
        ds = p * (dog @ v[keys].T)
        return tau * (ds @ k[keys]), tau * (ds.T @ qg), p.T @ dog, og, lse
    assert _fails_some_pin(monkeypatch, "group_backward", bad, [check_finite_differences, check_gradient_invariants])


def test_mutation_backward_transposed_dv(monkeypatch):
    def bad(qg, k, v, dog, keys):
        tau = 1.0 / np.sqrt(qg.shape[1])
        og, lse, p = O.group_forward(qg, k, v, keys)
        dvec = (dog * og).sum(axis=1)
        ds = p * (dog @ v[keys].T - dvec[:, None])
        return tau * (ds @ k[keys]), tau * (ds.T @ qg), (p / p.sum(axis=0, keepdims=True)).T @ dog, og, lse
    assert _fails_some_pin(monkeypatch, "group_backward", bad, [check_finite_differences, check_sparse_equals_masked_sdpa])


def test_mutation_merge_unweighted(monkeypatch):
    def bad(o_parts, lse_parts):   # averages the parts' outputs instead of weighting them by exp(LSE_p - LSE)
        lse = np.logaddexp.reduce(np.stack(lse_parts), axis=0)
        return sum(o_parts) / len(o_parts), lse
    assert _fails_some_pin(monkeypatch, "merge_states", bad,
                           [check_split_merge_equals_unsplit, check_merge_algebra]) > 0


def test_mutation_split_bounds_overlap(monkeypatch):
    def bad(k, n_split):           # parts overlap by one entry
        return [(max(0, s * k // n_split - 1), (s + 1) * k // n_split) for s in range(n_split)]
    assert _fails_some_pin(monkeypatch, "split_bounds", bad,
                           [check_split_bounds, check_split_merge_equals_unsplit]) > 0


def test_mutation_dense_missing_scale(monkeypatch):
    def bad(q_rows, k, v):
        logits = q_rows @ k.T
        m = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - m)
        return (w @ v) / w.sum(axis=1)[:, None], m[:, 0] + np.log(w.sum(axis=1))
    assert _fails_some_pin(monkeypatch, "dense_rows", bad, [check_dense_sdpa, check_dense_brute])


def test_mutation_dense_backward_missing_D(monkeypatch):
    def bad(q, k, v, do):
        tau = 1.0 / np.sqrt(q.shape[1])
        o, lse = O.dense_rows(q, k, v)
        p = np.exp(tau * (q @ k.T) - lse[:, None])
        ds = p * (do @ v.T)
        return tau * (ds @ k), tau * (ds.T @ q), p.T @ do
    assert _fails_some_pin(monkeypatch, "dense_backward_head", bad,
                           [check_dense_sdpa, check_dense_brute, check_dense_closed_forms])


def test_mutation_dense_backward_swapped_dq_dk(monkeypatch):
    def bad(q, k, v, do):
        tau = 1.0 / np.sqrt(q.shape[1])
        o, lse = O.dense_rows(q, k, v)
        p = np.exp(tau * (q @ k.T) - lse[:, None])
        ds = p * (do @ v.T - (do * o).sum(axis=1)[:, None])
        return tau * (ds.T @ q), tau * (ds @ k), p.T @ do
    assert _fails_some_pin(monkeypatch, "dense_backward_head", bad, [check_dense_sdpa, check_dense_brute])


def test_mutation_dense_blocks_chunk_local_lse(monkeypatch):
    # normalising P within the block instead of over all keys
    def bad(q, k, v, do, blocks, block=64, chunk=2048):
        tau = 1.0 / np.sqrt(q.shape[1])
        out = {}
        for j in blocks:
            keys = slice(j * block, (j + 1) * block)
            o, lse = O.dense_rows(q, k[keys], v[keys])
            p = np.exp(tau * (q @ k[keys].T) - lse[:, None])
            ds = p * (do @ v[keys].T - (do * o).sum(axis=1)[:, None])
            out[j] = (tau * (ds.T @ q), p.T @ do)
        return out
    assert _fails_some_pin(monkeypatch, "dense_dkdv_blocks", bad, [check_dense_sampled])


def test_mutation_dispatch_at_threshold(monkeypatch):
    def bad(k_per_head, n_blocks, threshold):
        return O.sparsity(k_per_head, n_blocks) >= threshold
    assert _fails_some_pin(monkeypatch, "use_sparse", bad, [check_dispatch_rule])


def test_mutation_pred_loss_no_centring(monkeypatch):
    def bad(q, k, wq, wk, group, block=64):
        tau = 1.0 / np.sqrt(q.shape[1])
        qbar, kbar = O.pool_mean(q, group), O.pool_mean(k, block)
        qhat, khat = qbar @ wq, kbar @ wk
        e = tau * (qhat @ khat.T) - tau * (qbar @ kbar.T)
        return float((e * e).mean()), e, qbar, kbar, qhat, khat
    assert _fails_some_pin(monkeypatch, "predictor_loss_head", bad,
                           [check_pred_loss_brute, check_pred_loss_closed_forms])


def test_mutation_pred_loss_centres_columns(monkeypatch):
    def bad(q, k, wq, wk, group, block=64):
        tau = 1.0 / np.sqrt(q.shape[1])
        qbar, kbar = O.pool_mean(q, group), O.pool_mean(k, block)
        qhat, khat = qbar @ wq, kbar @ wk
        diff = tau * (qhat @ khat.T) - tau * (qbar @ kbar.T)
        e = diff - diff.mean(axis=0, keepdims=True)
        return float((e * e).mean()), e, qbar, kbar, qhat, khat
    assert _fails_some_pin(monkeypatch, "predictor_loss_head", bad,
                           [check_pred_loss_brute, check_pred_loss_closed_forms])


def test_mutation_pred_grad_swapped(monkeypatch):
    def bad(q, k, wq, wk, group, block=64):
        tau = 1.0 / np.sqrt(q.shape[1])
        loss, e, qbar, kbar, qhat, khat = O.predictor_loss_head(q, k, wq, wk, group, block)
        ds = 2.0 * e / e.size
        return loss, tau * (kbar.T @ (ds.T @ qhat)), tau * (qbar.T @ (ds @ khat))
    assert _fails_some_pin(monkeypatch, "predictor_loss_grad_head", bad, [check_pred_loss_brute])


def test_mutation_pred_grad_half(monkeypatch):
    def bad(q, k, wq, wk, group, block=64):
        tau = 1.0 / np.sqrt(q.shape[1])
        loss, e, qbar, kbar, qhat, khat = O.predictor_loss_head(q, k, wq, wk, group, block)
        ds = e / e.size                       # the factor 2 of d(e^2) dropped
        return loss, tau * (qbar.T @ (ds @ khat)), tau * (kbar.T @ (ds.T @ qhat))
    assert _fails_some_pin(monkeypatch, "predictor_loss_grad_head", bad, [check_pred_loss_brute])


def test_mutation_coverage_inclusive(monkeypatch):
    def bad(scores_row, coverage, k_cap):       # stops one block late when a prefix lands exactly on the target
        nb = len(scores_row)
        s_ = np.asarray(scores_row)
        order = np.lexsort((np.arange(nb), -s_))
        cum = np.cumsum(O.block_mass(s_)[order])
        c = 1 + int(np.count_nonzero(cum <= coverage))
        return np.sort(order[:min(c, k_cap, nb)])
    assert _fails_some_pin(monkeypatch, "select_coverage_row", bad, [check_coverage_closed_forms])


def test_mutation_coverage_unnormalised(monkeypatch):
    def bad(scores_row):
        s_ = np.asarray(scores_row, dtype=np.float64)
        return np.exp(s_ - s_.max())
    assert _fails_some_pin(monkeypatch, "block_mass", bad, [check_coverage_brute, check_coverage_closed_forms])


def test_mutation_coverage_ties_high(monkeypatch):
    def bad(scores_row, coverage, k_cap):
        nb = len(scores_row)
        s_ = np.asarray(scores_row)
        order = np.lexsort((-np.arange(nb), -s_))
        cum = np.cumsum(O.block_mass(s_)[order])
        c = 1 + int(np.count_nonzero(cum < coverage))
        return np.sort(order[:min(c, k_cap, nb)])
    assert _fails_some_pin(monkeypatch, "select_coverage_row", bad, [check_coverage_brute, check_coverage_closed_forms])


def test_mutation_diagonal_off_by_one_group(monkeypatch):
    def bad(g, group, n_blocks, block=64):
        return np.arange((g + 1) * group // block, min((g + 2) * group // block, n_blocks))
    assert _fails_some_pin(monkeypatch, "diagonal_blocks", bad, [check_diagonal_brute])


def test_mutation_pooled_lse_without_mean(monkeypatch):
    orig = O.predict_head_pooled

    def bad(q, k, wq, wk, group, pooling, block=64):   # log-sum-exp instead of log-mean-exp
        out = orig(q, k, wq, wk, group, pooling, block)
        return out + math.log(group * block) if pooling == "lse" else out
    assert _fails_some_pin(monkeypatch, "predict_head_pooled", bad, [check_pooled_scores_brute])


def test_mutation_select_rows_ties_to_highest_id(monkeypatch):
    def bad(scores, k):
        s = np.asarray(scores)[:, ::-1]
        order = np.argsort(-s, axis=1, kind="stable")[:, :k]
        return np.sort(s.shape[1] - 1 - order, axis=1)
    monkeypatch.setattr(O, "select_rows", bad)
    with pytest.raises(AssertionError):
        check_select_rows_vectorised()


def test_mutation_reverse_csr_groups_unsorted(monkeypatch):
    real = O.reverse_index_csr

    def bad(idx_bh, n_blocks):
        ptr, groups = real(idx_bh, n_blocks)
        out = groups.copy()
        for j in range(n_blocks):
            out[ptr[j]:ptr[j + 1]] = out[ptr[j]:ptr[j + 1]][::-1]
        return ptr, out
    monkeypatch.setattr(O, "reverse_index_csr", bad)
    with pytest.raises(AssertionError):
        check_reverse_index_csr()


def test_mutation_block_part_without_D(monkeypatch):
    def bad(q, k, v, do, idx_row, group, g, j, block=64):
        tau = 1.0 / np.sqrt(q.shape[1])
        rows = slice(g * group, (g + 1) * group)
        _, lse, _ = O.group_forward(q[rows], k, v, O.kept_keys(idx_row, block))
        kj, vj = k[j * block:(j + 1) * block], v[j * block:(j + 1) * block]
        p = np.exp(tau * (q[rows] @ kj.T) - lse[:, None])
        ds = p * (do[rows] @ vj.T)
        return tau * (ds.T @ q[rows]), p.T @ do[rows]
    monkeypatch.setattr(O, "dkdv_block_part", bad)
    with pytest.raises(AssertionError):
        check_dkdv_block_part()


def test_mutation_backward_dk_without_tau(monkeypatch):
    def bad(qg, k, v, dog, keys):   # dK misses the logit scale tau = 1/sqrt(d) that dQ keeps
        tau = 1.0 / np.sqrt(qg.shape[1])
        og, lse, p = O.group_forward(qg, k, v, keys)
        dvec = (dog * og).sum(axis=1)
        ds = p * (dog @ v[keys].T - dvec[:, None])
        return tau * (ds @ k[keys]), ds.T @ qg, p.T @ dog, og, lse
    assert _fails_some_pin(monkeypatch, "group_backward", bad, [check_finite_differences,
                                                                 check_sparse_equals_masked_sdpa])


def test_mutation_backward_dq_tau_twice(monkeypatch):
    def bad(qg, k, v, dog, keys):   # dQ scaled by tau^2
        tau = 1.0 / np.sqrt(qg.shape[1])
        og, lse, p = O.group_forward(qg, k, v, keys)
        dvec = (dog * og).sum(axis=1)
        ds = p * (dog @ v[keys].T - dvec[:, None])
        return tau * tau * (ds @ k[keys]), tau * (ds.T @ qg), p.T @ dog, og, lse
    assert _fails_some_pin(monkeypatch, "group_backward", bad, [check_finite_differences,
                                                                 check_sparse_equals_masked_sdpa])


def test_mutation_backward_dv_unnormalised(monkeypatch):
    def bad(qg, k, v, dog, keys):   # dV from exp(logits - row max) instead of the normalised P
        tau = 1.0 / np.sqrt(qg.shape[1])
        og, lse, p = O.group_forward(qg, k, v, keys)
        logits = tau * (qg @ k[keys].T)
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        dvec = (dog * og).sum(axis=1)
        ds = p * (dog @ v[keys].T - dvec[:, None])
        return tau * (ds @ k[keys]), tau * (ds.T @ qg), e.T @ dog, og, lse
    assert _fails_some_pin(monkeypatch, "group_backward", bad, [check_finite_differences,
                                                                 check_sparse_equals_masked_sdpa])
