"""Selection with each group's own KV blocks forced (DSA_SELECT_DIAGONAL), top-k and
coverage rules, on the GPU against the float64 oracle applied to the GPU's own scores;
attention over the resulting lists against the oracle."""
import json

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_qk_amd as dsa
import oracle
import synth
from tests import parity as P
from tests.parity import f64
from tests.test_coverage_gpu import COVER_TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


def _wl(grid, heads, d, group, k, rank=16, streamed=False, seed=83):
    return synth.Workload(f"diag_{grid}_{heads}_{d}_{group}_{k}", seed, 1, heads, d, grid, 8, 3.0, rank, group, k=k,
                          backward=True, streamed=streamed)


def _run(inp, coverage):
    w = inp.workload
    p = P.problem_of(w, heads=inp.q.shape[1])
    plan = dsa.SparseAttentionPlan(p, inp.k_per_head, materialise_scores=not w.streamed, coverage=coverage,
                                   select_flags=dsa.SELECT_DIAGONAL)
    dev = {n: P.to_device(getattr(inp, n)) for n in ("q", "k", "v", "do")}
    W = P.to_device(inp.w)
    plan.idx.zero_()
    plan.rev_idx.zero_()
    plan.predict(dev["q"], dev["k"], W, W)
    dump = None if not w.streamed else torch.empty(p.batch, p.heads, p.n_groups, p.n_blocks, dtype=torch.float32,
                                                   device="cuda")
    plan.select(scores_dump=dump)
    torch.cuda.synchronize()
    scores = (plan.scores if not w.streamed else dump).cpu().numpy()
    idx = plan.idx.cpu().numpy()
    cnt = plan.cnt.cpu().numpy() if plan.cnt is not None else None
    rows = []
    for h in range(p.heads):
        k = plan.k_per_head[h]
        base = int(plan.row_base[h])
        full = idx[base:base + p.n_groups * k].reshape(p.n_groups, k)
        r = [full[g, :(cnt[0, h, g] if cnt is not None else k)].astype(np.int64) for g in range(p.n_groups)]
        for g, x in enumerate(r):      # host check before the attention kernels read the lists
            assert x.min() >= 0 and x.max() < p.n_blocks and (np.diff(x) > 0).all(), (h, g)
        rows.append(r)
    plan.forward(dev["q"], dev["k"], dev["v"])
    plan.backward(dev["q"], dev["k"], dev["v"], dev["do"])
    torch.cuda.synchronize()
    return plan, scores, rows


CASES = [
    ("g64_k3", _wl((2, 16, 32), 2, 64, 64, 3), None),
    ("g128_k4", _wl((3, 16, 32), 2, 128, 128, 4, rank=32), None),
    ("g128_k2_forced_only", _wl((2, 16, 16), 2, 64, 128, 2), None),
    ("g64_streamed_k5", _wl((2, 16, 32), 2, 64, 64, 5, streamed=True), None),
    ("g128_cov0.5_cap6", _wl((3, 16, 32), 2, 128, 128, 6, rank=32), 0.5),
    ("g64_cov0.9_cap24", _wl((2, 32, 32), 2, 64, 64, 24), 0.9),
]


@pytest.mark.parametrize("name,w,cov", CASES, ids=[c[0] for c in CASES])
def test_diagonal_parity(name, w, cov):
    print(f"CASE {name} N={w.seq_len} H={w.heads} d={w.head_dim} G={w.group} k={w.k} cov={cov}", flush=True)
    inp = synth.generate(w)
    plan, scores, rows = _run(inp, cov)
    p = plan.p
    flips = 0
    for h in range(p.heads):
        cap = plan.k_per_head[h]
        for g in range(p.n_groups):
            s = scores[0, h, g]
            got = rows[h][g]
            own = oracle.diagonal_blocks(g, p.group, p.n_blocks)
            assert np.isin(own, got).all(), (h, g)
            # given its count, the row is the forced blocks plus the best of the rest
            assert np.array_equal(got, oracle.select_row_diag(s, len(got), g, p.group)), (h, g)
            if cov is None:
                assert len(got) == cap
            else:
                want = len(oracle.select_coverage_row_diag(s, cov, cap, g, p.group))
                if len(got) != want:
                    flips += 1
                    cum = np.cumsum(oracle.block_mass(s)[oracle.select_order(s, own)])
                    c = len(got)
                    assert c == cap or cum[c - 1] >= cov - COVER_TOL, (h, g, c, want)
                    assert c == len(own) or cum[c - 2] < cov + COVER_TOL, (h, g, c, want)
    rep = P.Report()
    for h in range(p.heads):
        q, k, v, do = (f64(getattr(inp, n)[0, h]) for n in ("q", "k", "v", "do"))
        o, lse = oracle.forward_head(q, k, v, rows[h], p.group)
        dq, dk, dv = oracle.backward_head(q, k, v, do, rows[h], p.group)
        for n_, got, ref in (("O", plan.O, o), ("LSE", plan.LSE, lse), ("dQ", plan.dQ, dq), ("dK", plan.dK, dk),
                             ("dV", plan.dV, dv)):
            rep.add(n_, got[0, h].cpu().numpy(), ref)
    print("DIAG " + json.dumps({"case": name, "near_tie_rows": flips, **rep.summary()}), flush=True)
    P.assert_float_parity(rep, bf16=True)
