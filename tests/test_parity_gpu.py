"""GPU parity of the HIP hot path against the float64 oracle (needs an MI355X).

Small clustered cases span several tiles and ragged tails (NB not a multiple
of 64, per-head ragged k, empty reverse lists) and are checked element by
element; the full-size workloads are checked on every kept-block row where
cheap and on seeded samples of rows and blocks for the float outputs.
"""
from __future__ import annotations

import functools
import json

import numpy as np
import pytest
import torch

import oracle
import synth
import dynamic_sparse_attention_qk_amd as dsa
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


def _wl(grid, heads, d, group, k=None, rank=16, dtype="bf16", backward=True, centres=8, seed=77, kph=None,
        batch=1, order="morton"):
    w = synth.Workload(f"small_{grid}_{heads}_{d}_{group}_{batch}_{order}", seed, batch, heads, d, grid, centres, 3.0,
                       rank, group, k=k, dtype=dtype, backward=backward, order=order)
    return w


def _inputs(w, kph=None):
    inp = synth.generate(w)
    if kph is not None:
        inp.k_per_head = np.asarray(kph, dtype=np.int32)
    return inp


def _print(name, rep, extra=None):
    rec = {"case": name, "score_err": rep.score_err, "idx_rows": rep.idx_rows,
           "idx_rows_own_scores_differ": rep.idx_own_mismatch, "errs": rep.summary()}
    if extra:
        rec.update(extra)
    print("PARITY " + json.dumps(rec), flush=True)


SMALL = [
    # name, workload, per-head k override
    ("cfg1_fp32_fwd", synth.workload(1), None),
    ("d64_g64_nb24", _wl((4, 16, 24), 3, 64, 64, k=5), None),
    ("d128_g64_nb30", _wl((4, 20, 24), 2, 128, 64, k=7, rank=32), None),
    ("d128_g128_nb32", _wl((8, 16, 16), 2, 128, 128, k=6, rank=32), None),
    ("d64_g64_nb70", _wl((4, 28, 40), 2, 64, 64, k=9, rank=8), None),
    ("d128_ragged_heads", _wl((4, 16, 32), 4, 128, 64, k=1, rank=64), [1, 3, 32, 9]),
    ("d64_g128_k1", _wl((4, 16, 32), 2, 64, 128, k=1, rank=16), None),
    ("batch3_ragged_heads", _wl((2, 16, 32), 3, 128, 64, k=4, rank=32, batch=3), [2, 7, 4]),
    ("batch2_fp32_fwd", _wl((2, 16, 16), 2, 64, 64, k=3, dtype="f32", backward=False, batch=2), None),
    # cube-ordered tokens: every group an aligned 4x4x4 (4x4x8) box; rows y = 20, 21 are partial-edge groups
    ("cubes_g64_edge_rows", _wl((4, 22, 24), 2, 128, 64, k=7, rank=32, order="cubes"), None),
    ("cubes_g128", _wl((8, 16, 16), 2, 128, 128, k=6, rank=32, order="cubes"), None),
]


@pytest.mark.parametrize("name,w,kph", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(name, w, kph):
    print(f"CASE {name} N={w.seq_len} H={w.heads} d={w.head_dim} G={w.group}", flush=True)
    inp = _inputs(w, kph)
    run = P.run_gpu(inp)
    rep = P.Report()
    P.check_predict_select(run, rep)
    P.check_forward(run, rep)
    if w.backward:
        P.check_backward(run, rep)
    _print(name, rep)
    P.assert_float_parity(rep, bf16=(w.dtype == "bf16"))


@pytest.mark.parametrize("case", ["d128_g64", "d64_g128"])
def test_streamed_select_matches_materialised(case):
    if case == "d128_g64":
        w, kph = _wl((4, 16, 40), 3, 128, 64, k=4, rank=32), [4, 1, 40]
    else:
        w, kph = _wl((8, 16, 40), 2, 64, 128, k=11, rank=16), None
    inp = _inputs(w, kph)
    a = P.run_gpu(inp, materialise=True, backward=False)
    b = P.run_gpu(inp, materialise=False, backward=False, dump=True)
    np.testing.assert_array_equal(a.host["scores"].view(np.uint32), b.host["scores"].view(np.uint32))
    n = int(a.plan.row_base[-1])
    np.testing.assert_array_equal(a.host["idx"][:n], b.host["idx"][:n])
    np.testing.assert_array_equal(a.host["rev_ptr"], b.host["rev_ptr"])
    np.testing.assert_array_equal(a.host["rev_idx"][:n], b.host["rev_idx"][:n])
    np.testing.assert_array_equal(a.plan.O.cpu().numpy(), b.plan.O.cpu().numpy())


def test_dense_selection_equals_full_attention():
    # k = NB: every block kept, so the sparse path is plain attention
    w = _wl((4, 16, 16), 2, 128, 64, k=16, rank=32)
    inp = _inputs(w)
    run = P.run_gpu(inp)
    p = run.plan.p
    for h in range(p.heads):
        assert (run.idx_rows(0, h) == np.arange(16)[None, :]).all()
    q, k, v, do = (torch.tensor(P.f64(getattr(inp, n)[0])) for n in ("q", "k", "v", "do"))
    q.requires_grad_(True), k.requires_grad_(True), v.requires_grad_(True)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    (ref * do).sum().backward()
    rep = P.Report()
    rep.add("O", run.plan.O.cpu().numpy()[0], ref.detach().numpy())
    rep.add("dQ", run.plan.dQ.cpu().numpy()[0], q.grad.numpy())
    rep.add("dK", run.plan.dK.cpu().numpy()[0], k.grad.numpy())
    rep.add("dV", run.plan.dV.cpu().numpy()[0], v.grad.numpy())
    _print("dense_k_eq_nb", rep)
    P.assert_float_parity(rep, bf16=True)


def _select_only(scores: np.ndarray, kph, group=64):
    B, H, NG, NB = scores.shape
    p = dsa.Problem(batch=B, heads=H, seq_len=NB * 64, head_dim=64, rank=16, group=group)
    plan = dsa.SparseAttentionPlan(p, kph, backward=False)
    plan.scores.copy_(torch.from_numpy(scores))
    plan.select()
    torch.cuda.synchronize()
    return plan


def test_select_ties_and_signed_zeros():
    rng = np.random.default_rng(5)
    NB, NG = 100, 8 * 4  # G=64 -> N = 6400, NG = 100; use 100 rows
    vals = np.array([0.0, -0.0, 1.0, -1.0, 2.5, 1e-38, -1e-38, 3.0e38, -3.0e38, 7.0], dtype=np.float32)
    scores = rng.choice(vals, size=(1, 2, 100, NB)).astype(np.float32)
    scores[0, 1, :50] = rng.standard_normal((50, NB)).astype(np.float32)
    scores[0, 1, 50:] = np.float32(0.0)
    scores[0, 1, 50:, ::3] = np.float32(-0.0)
    kph = [17, 33]
    plan = _select_only(scores, kph)
    idx = plan.idx.cpu().numpy()
    for h in range(2):
        rows = idx[int(plan.row_base[h]): int(plan.row_base[h]) + 100 * kph[h]].reshape(100, kph[h])
        for g in range(100):
            assert np.array_equal(rows[g], oracle.select_row(scores[0, h, g].astype(np.float64), kph[h])), (h, g)


def test_select_extremes_k1_and_knb():
    rng = np.random.default_rng(6)
    NB = 130
    scores = rng.standard_normal((1, 2, NB, NB)).astype(np.float32)
    scores[0, 0, 3] = 1.0  # constant row: the lowest ids win
    kph = [1, NB]
    plan = _select_only(scores, kph)
    idx = plan.idx.cpu().numpy()
    r0 = idx[:NB]
    assert r0[3] == 0
    assert np.array_equal(r0, np.array([oracle.select_row(scores[0, 0, g].astype(np.float64), 1)[0] for g in range(NB)]))
    r1 = idx[NB: NB + NB * NB].reshape(NB, NB)
    assert (r1 == np.arange(NB)[None, :]).all()
    # reverse index: with k = NB every block lists every group
    rp = plan.rev_ptr.cpu().numpy()[1]
    assert (np.diff(rp) == NB).all()


def test_deterministic_bitwise():
    w = _wl((4, 16, 24), 2, 128, 64, k=5, rank=32)
    inp = _inputs(w)
    a = P.run_gpu(inp)
    b = P.run_gpu(inp)
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        x, y = getattr(a.plan, name).cpu().numpy(), getattr(b.plan, name).cpu().numpy()
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


def test_unkept_blocks_get_zero_gradient():
    # k = 1 of 32 blocks with clustered keys: several blocks are kept by no group
    w = _wl((4, 16, 32), 2, 64, 64, k=1)
    inp = _inputs(w)
    run = P.run_gpu(inp)
    dK, dV = run.plan.dK.cpu().numpy(), run.plan.dV.cpu().numpy()
    for h in range(2):
        unkept = sorted(set(range(32)) - set(np.unique(run.idx_rows(0, h)).tolist()))
        assert unkept, "expected at least one block kept by no group"
        assert (np.diff(run.host["rev_ptr"][h])[unkept] == 0).all()
        for j in unkept:
            assert (dK[0, h, 64 * j:64 * (j + 1)] == 0).all() and (dV[0, h, 64 * j:64 * (j + 1)] == 0).all()
    rep = P.Report()
    P.check_backward(run, rep)
    P.assert_float_parity(rep, bf16=True)


# ------------------------------------------------------------------ full-size workloads, whole

@functools.lru_cache(maxsize=1)
def _full_run(cid):
    """The workload's inputs and one GPU pass (predict, select, fwd, bwd), kept for the tests of that workload."""
    w = synth.workload(cid)
    print(f"CASE full workload {cid} ({w.name}) N={w.seq_len} heads={w.heads}", flush=True)
    inp = synth.generate(w, threads=16)
    run = P.run_gpu(inp, materialise=not w.streamed, dump=w.streamed, scores_on_device=True)
    return w, run


@pytest.mark.parametrize("cid,heads", [(2, None), (3, range(0, 12)), (3, range(12, 24)), (4, range(0, 12)),
                                       (4, range(12, 24))],
                         ids=["w2_all_heads", "w3_heads_0_11", "w3_heads_12_23", "w4_heads_0_11", "w4_heads_12_23"])
def test_full_workload_every_element(cid, heads):
    """Every row's scores, kept ids and reverse lists, and every element of O, LSE (and dQ, dK, dV for the
    training workloads) of the listed heads, against the oracle run with the GPU's lists."""
    w, run = _full_run(cid)
    hl = None if heads is None else list(heads)
    rep = P.Report()
    P.check_selection_full(run, rep, heads=hl)
    P.check_attention_full(run, rep, heads=hl)
    _print(f"full_{cid}" + ("" if hl is None else f"_heads_{hl[0]}_{hl[-1]}"), rep,
           {"k_per_head": sorted(set(int(x) for x in run.inp.k_per_head)), "every_element": True})
    P.assert_float_parity(rep, bf16=True)
