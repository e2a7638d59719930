"""GPU parity of the 520,000-token workload (24 heads, per-head kept counts 194..1,904 of 8,125 blocks,
streamed block scores) against the float64 oracle.

One GPU pass of the whole layer (predict, streamed select with the scores dumped for checking, forward,
backward) is shared by the tests below, each bounded to about a minute of host time:
  - every selection row of every head: scores within the row-relative bound, the oracle's top-k of the GPU's
    scores equal to the GPU's ids bit for bit, the reverse index exact;
  - O, LSE and dQ on a seeded 2% of the query groups of every head;
  - dK and dV on whole reverse lists: the heaviest head's median-length and longest lists (about 1,950 and
    3,100 groups), the lightest head's longest list and a middle head's median one.
The float oracle of a group needs its softmax over all its kept keys (up to 121,856), so the long lists are
spread over threads (tests/parity.py).
"""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import oracle
import synth
import dynamic_sparse_attention_qk_amd as dsa
from tests import parity as P

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def w5():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()
    w = synth.workload(5)
    print(f"CASE full workload 5 ({w.name}) N={w.seq_len} heads={w.heads}", flush=True)
    inp = synth.generate(w, threads=16)
    run = P.run_gpu(inp, materialise=False, dump=True, scores_on_device=True)
    yield w, run
    del run
    torch.cuda.empty_cache()


def _print(name, rep, extra=None):
    rec = {"case": name, "score_err": rep.score_err, "idx_rows": rep.idx_rows,
           "idx_rows_own_scores_differ": rep.idx_own_mismatch, "errs": rep.summary()}
    rec.update(extra or {})
    print("PARITY " + json.dumps(rec), flush=True)


def test_520k_selection_every_row(w5):
    w, run = w5
    rep = P.Report()
    P.check_selection_full(run, rep)
    assert rep.idx_rows == w.heads * w.n_groups
    _print("full_5_selection", rep, {"k_per_head": [int(x) for x in run.inp.k_per_head]})


@pytest.mark.parametrize("heads", [range(0, 12), range(12, 24)], ids=["heads_0_11", "heads_12_23"])
def test_520k_forward_dq_sampled_groups(w5, heads):
    """O, LSE and dQ of 2% of the groups of each head (seeded; the first and last group always)."""
    w, run = w5
    p = run.plan.p
    rng = np.random.default_rng(1005 + heads[0])
    n = max(2, int(np.ceil(0.02 * p.n_groups)))
    jobs = []
    for h in heads:
        gl = sorted(set([0, p.n_groups - 1] + rng.choice(p.n_groups, size=n, replace=False).tolist()))
        jobs += [(h, g) for g in gl]
    inp = run.inp
    head_in = {h: tuple(P.f64(getattr(inp, t)[0, h]) for t in ("q", "k", "v", "do")) for h in heads}
    idx = {h: run.idx_rows(0, h) for h in heads}

    def one(job):
        h, g = job
        q, k, v, do = head_in[h]
        rows = slice(g * p.group, (g + 1) * p.group)
        dq, _, _, og, lse = oracle.group_backward(q[rows], k, v, do[rows], oracle.kept_keys(idx[h][g]))
        return h, g, og, lse, dq

    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    rep = P.Report()
    outs = {h: {n_: run.out_head(n_, 0, h) for n_ in ("O", "LSE", "dQ")} for h in heads}
    with threadpool_limits(1), ThreadPoolExecutor(P._pool_threads()) as ex:
        for h, g, og, lse, dq in ex.map(one, jobs):
            rows = slice(g * p.group, (g + 1) * p.group)
            rep.add("O", outs[h]["O"][rows], og)
            rep.add("LSE", outs[h]["LSE"][rows], lse)
            rep.add("dQ", outs[h]["dQ"][rows], dq)
    _print(f"full_5_fwd_dq_heads_{heads[0]}_{heads[-1]}", rep, {"groups_checked": len(jobs)})
    P.assert_float_parity(rep, bf16=True)


def _lists_of(run, h):
    p = run.plan.p
    rp = run.host["rev_ptr"][h]
    base = int(run.plan.row_base[h])
    return rp, base, np.diff(rp)


@pytest.mark.parametrize("which", ["heaviest_median", "heaviest_longest", "lightest_longest_and_middle_median"])
def test_520k_dkdv_whole_reverse_lists(w5, which):
    w, run = w5
    p = run.plan.p
    kph = np.asarray(run.inp.k_per_head)
    order = np.argsort(kph, kind="stable")
    heavy, light, mid = int(order[-1]), int(order[0]), int(order[len(order) // 2])
    picks = []
    for h, how in {"heaviest_median": [(heavy, "median")], "heaviest_longest": [(heavy, "longest")],
                   "lightest_longest_and_middle_median": [(light, "longest"), (mid, "median")]}[which]:
        rp, base, lens = _lists_of(run, h)
        j = int(np.argmax(lens)) if how == "longest" else int(np.argsort(lens, kind="stable")[len(lens) // 2])
        picks.append((h, j, int(lens[j])))
    rep = P.Report()
    for h, j, ln in picks:
        rp, base, _ = _lists_of(run, h)
        groups = run.host["rev_idx"][base + rp[j]: base + rp[j + 1]]
        assert len(groups) == ln and ln > 0
        inp = run.inp
        q, k, v, do = (P.f64(getattr(inp, t)[0, h]) for t in ("q", "k", "v", "do"))
        dk, dv = P.dkdv_block_threaded(q, k, v, do, run.idx_rows(0, h), p.group, j, groups)
        rep.add("dK", run.out_head("dK", 0, h)[j * 64:(j + 1) * 64], dk)
        rep.add("dV", run.out_head("dV", 0, h)[j * 64:(j + 1) * 64], dv)
    _print(f"full_5_dkdv_{which}", rep, {"lists": [{"head": h, "k_h": int(kph[h]), "block": j, "groups": ln}
                                                   for h, j, ln in picks]})
    P.assert_float_parity(rep, bf16=True)
