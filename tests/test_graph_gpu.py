"""The whole hot path (predict, select, forward, backward) captured in one HIP graph:
every replay, with eager work and synchronisations between replays, must reproduce the
eager run bit for bit.  The library allocates nothing and issues no memset, so its calls
capture as they are."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_qk_amd as dsa
import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


OUTS = ("qhat", "khat", "scores", "idx", "rev_ptr", "rev_idx", "O", "LSE", "dQ", "dK", "dV")


@pytest.mark.parametrize("coverage", [None, 0.9])
def test_step_graph_replays_match_eager(coverage):
    w = synth.Workload("graph_small", 91, 1, 3, 128, (2, 16, 32), 8, 3.0, 32, 64, k=5, backward=True)
    inp = synth.generate(w)
    p = P.problem_of(w)
    plan = dsa.SparseAttentionPlan(p, inp.k_per_head, coverage=coverage)
    Q, K, V, W, dO = (P.to_device(getattr(inp, n)) for n in ("q", "k", "v", "w", "do"))
    plan.idx.zero_()
    plan.rev_idx.zero_()
    plan.step(Q, K, V, W, W, dO)
    torch.cuda.synchronize()
    names = OUTS + (("cnt",) if coverage is not None else ())
    ref = {n: getattr(plan, n).clone() for n in names}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.step(Q, K, V, W, W, dO)              # warm-up on the capture stream's side, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.step(Q, K, V, W, W, dO)
    for rep in range(3):
        for n in names:                           # eager work between replays: poison every output
            t = getattr(plan, n)
            t.fill_(float("nan") if t.is_floating_point() else -7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            got, want = getattr(plan, n), ref[n]
            if n == "rev_idx" and coverage is not None:
                # with per-row counts each (b, h) region of the reverse list is filled only up to its total
                rp = ref["rev_ptr"].cpu().numpy()
                for bh in range(p.batch * p.heads):
                    a, e = int(plan.row_base[bh]), int(plan.row_base[bh]) + int(rp[bh, -1])
                    assert torch.equal(got[a:e], want[a:e]), (rep, n, bh)
                continue
            if got.is_floating_point():
                assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (rep, n)
            else:
                assert torch.equal(got, want), (rep, n)
