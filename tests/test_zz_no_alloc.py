"""The selection call without a workspace (static per-GPU scratch) against the one with a workspace.

dsa_select_topk_blocks_noalloc must give the same kept-block lists and reverse
index, bit for bit, as dsa_select_topk_blocks on the same scores; two calls in a
row, the second on a smaller problem, so the second runs on scratch the first
left behind (its counters must be cleared by the call itself).
"""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import synth
import dynamic_sparse_attention_qk_amd as dsa
from synth.device import problem_of, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


def _selections(w, heads=None):
    inp = synth.generate(w, heads=heads)
    p = problem_of(w, heads=inp.q.shape[1])
    kph = [int(x) for x in inp.k_per_head]
    assert dsa.workspace_bytes(p, kph, dsa.DSA_WS_SELECT) <= dsa.NOALLOC_SCRATCH_BYTES
    plan = dsa.SparseAttentionPlan(p, kph, materialise_scores=not w.streamed, backward=False)
    Q, K, W = to_device(inp.q), to_device(inp.k), to_device(inp.w)
    plan.predict(Q, K, W, W)
    # reference: the call with a caller workspace
    plan.idx.fill_(-7)
    plan.rev_idx.fill_(-7)
    plan.rev_ptr.fill_(-7)
    plan.select()
    torch.cuda.synchronize()
    n = int(plan.row_base[-1])
    ref = {"idx": plan.idx[:n].cpu().numpy(), "rev_ptr": plan.rev_ptr.cpu().numpy(),
           "rev_idx": plan.rev_idx[:n].cpu().numpy()}
    assert ref["idx"].min() >= 0 and ref["idx"].max() < p.n_blocks
    # the same selection through the entry point without a workspace, into poisoned outputs
    idx = torch.full_like(plan.idx, -3)
    rev_ptr = torch.full_like(plan.rev_ptr, -3)
    rev_idx = torch.full_like(plan.rev_idx, -3)
    dsa.select_topk_blocks_noalloc(p, plan.scores, plan.qhat, plan.khat, kph, idx, rev_ptr, rev_idx)
    torch.cuda.synchronize()
    got = {"idx": idx[:n].cpu().numpy(), "rev_ptr": rev_ptr.cpu().numpy(), "rev_idx": rev_idx[:n].cpu().numpy()}
    return p, ref, got


def test_noalloc_select_equals_workspace_select_twice():
    # first the 57,600-token layer (24 heads, k = 90, ~7.9 MB of scratch), then a smaller, streamed one
    cases = [synth.workload(3).with_(backward=False),
             synth.Workload("small_streamed", 4243, 1, 3, 128, (4, 16, 40), 8, 3.0, 32, 64, k=7, backward=False,
                            streamed=True)]
    for w in cases:
        p, ref, got = _selections(w)
        for name in ("idx", "rev_ptr", "rev_idx"):
            np.testing.assert_array_equal(got[name], ref[name], err_msg=f"{w.name}: {name}")
        print("NOALLOC " + json.dumps({"case": w.name, "tokens": p.seq_len, "heads": p.heads,
                                       "list_entries": int(ref["idx"].size), "bitwise_equal": True}), flush=True)
