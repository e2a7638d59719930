"""Block scores pooled from the token-level low-rank logits (max, log-mean-exp) on the
GPU against the float64 oracle, and the top-k selection on them (ids bit-exact given
the GPU's own scores)."""
import json

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_qk_amd as dsa
import oracle
import synth
from tests import parity as P
from tests.parity import f64

pytestmark = pytest.mark.gpu

POOL = {"max": dsa.POOL_MAX, "lse": dsa.POOL_LSE}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


def _wl(grid, heads, d, group, rank, k, dtype="bf16", seed=87):
    return synth.Workload(f"pool_{grid}_{heads}_{d}_{group}_{rank}_{dtype}", seed, 1, heads, d, grid, 8, 3.0, rank,
                          group, k=k, dtype=dtype, backward=False)


def _scores(inp, pooling):
    w = inp.workload
    p = P.problem_of(w, heads=inp.q.shape[1])
    Q, K, W = (P.to_device(x) for x in (inp.q, inp.k, inp.w))
    scores = torch.empty(p.batch, p.heads, p.n_groups, p.n_blocks, dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.workspace_bytes(p, None, dsa.DSA_WS_PRED_POOLED), dtype=torch.uint8, device="cuda")
    dsa.predict_block_scores_pooled(p, Q, K, W, W, POOL[pooling], scores, ws)
    torch.cuda.synchronize()
    return p, scores


def _row_err(got, ref):
    return float(np.max(np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)))


CASES = [
    ("fp32_d64_g64_r16", _wl((4, 16, 16), 2, 64, 64, 16, 4, dtype="f32")),
    ("bf16_d128_g128_r8", _wl((4, 16, 32), 2, 128, 128, 8, 5)),
    ("bf16_d64_g64_r64", _wl((2, 32, 32), 2, 64, 64, 64, 6)),
    ("bf16_d128_g64_r32_nb150", _wl((6, 40, 40), 2, 128, 64, 32, 9)),      # 150 blocks: a partial last chunk
]


@pytest.mark.parametrize("pooling", ["max", "lse"])
@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_pooled_scores_parity(name, w, pooling):
    print(f"CASE {name} {pooling} N={w.seq_len} H={w.heads} d={w.head_dim} r={w.rank} G={w.group}", flush=True)
    inp = synth.generate(w)
    p, scores = _scores(inp, pooling)
    got = scores.cpu().numpy()
    err = 0.0
    for h in range(p.heads):
        wq = inp.w[h].astype(np.float64)
        ref = oracle.predict_head_pooled(f64(inp.q[0, h]), f64(inp.k[0, h]), wq, wq, p.group, pooling)
        err = max(err, _row_err(got[0, h], ref))
    # top-k on the GPU's own scores: bit-exact against the oracle's rule on the same scores
    kph = list(inp.k_per_head)
    plan = dsa.SparseAttentionPlan(p, kph, backward=False)
    plan.scores.copy_(scores)
    plan.select()
    torch.cuda.synchronize()
    idx = plan.idx.cpu().numpy()
    for h in range(p.heads):
        rows = idx[int(plan.row_base[h]):int(plan.row_base[h]) + p.n_groups * kph[h]].reshape(p.n_groups, kph[h])
        want = np.stack([oracle.select_row(got[0, h, g], kph[h]) for g in range(p.n_groups)])
        assert np.array_equal(rows, want), h
    print("POOLED " + json.dumps({"case": name, "pooling": pooling, "score_row_err": err}), flush=True)
    assert err <= P.SCORE_TOL


@pytest.mark.parametrize("pooling", ["max", "lse"])
def test_pooled_scores_full_57k(pooling):
    """57,600 tokens, d = 128, r = 32: sampled groups of two heads against the oracle."""
    w = synth.workload(3).with_(backward=False)
    inp = synth.generate(w, heads=[0, 23])
    p, scores = _scores(inp, pooling)
    got = scores.cpu().numpy()
    err = 0.0
    for h in range(p.heads):
        wq = inp.w[h].astype(np.float64)
        for g, ref in oracle.predict_head_pooled_groups(f64(inp.q[0, h]), f64(inp.k[0, h]), wq, wq, p.group, pooling,
                                                        [0, 449, 899]).items():
            err = max(err, _row_err(got[0, h, g][None], ref[None]))
    print("POOLED " + json.dumps({"case": "full_57k", "pooling": pooling, "score_row_err": err}), flush=True)
    assert err <= P.SCORE_TOL
