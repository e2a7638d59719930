"""Dense attention (the dispatcher's branch for layers whose sparsity is at or below
the threshold) on the GPU against the float64 oracle's full attention, and against
the sparse path with every block kept, which must give the same bits."""
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


def _wl(grid, heads, d, group, rank=16, dtype="bf16", backward=True, seed=71, batch=1):
    nb = grid[0] * grid[1] * grid[2] // 64
    return synth.Workload(f"dense_{grid}_{heads}_{d}_{group}_{dtype}_{batch}", seed, batch, heads, d, grid, 8, 3.0,
                          rank, group, k=nb, dtype=dtype, backward=backward)


CASES = [
    ("cfg1_fp32_fwd", synth.workload(1).with_(k=16, keep=None)),
    ("fp32_d128_g128_fwd", _wl((3, 16, 32), 2, 128, 128, dtype="f32", backward=False)),
    ("d64_g64", _wl((2, 32, 32), 2, 64, 64)),
    ("d128_g128", _wl((3, 16, 32), 2, 128, 128, rank=32)),
    ("d128_g64_one_block", _wl((1, 8, 8), 3, 128, 64, rank=8)),
    ("d64_g128_two_blocks", _wl((1, 8, 16), 2, 64, 128)),
    ("d128_g64_ragged_tail", _wl((5, 8, 24), 2, 128, 64, rank=64)),   # 15 blocks: a partial last 8-block wave
    ("batch2_d64_g128", _wl((2, 16, 16), 2, 64, 128, batch=2)),
]


def _dense(inp, p, backward):
    plan = dsa.DenseAttentionPlan(p, backward=backward)
    dev = {n: P.to_device(getattr(inp, n)) for n in ("q", "k", "v")}
    plan.forward(dev["q"], dev["k"], dev["v"])
    if backward:
        dev["do"] = P.to_device(inp.do)
        plan.backward(dev["q"], dev["k"], dev["v"], dev["do"])
    torch.cuda.synchronize()
    return plan


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_dense_parity(name, w):
    print(f"CASE {name} N={w.seq_len} H={w.heads} d={w.head_dim} G={w.group} {w.dtype} bwd={w.backward}",
          flush=True)
    inp = synth.generate(w)
    p = P.problem_of(w)
    assert dsa.choose_path(p, [p.n_blocks] * p.heads, 0.0) == dsa.PATH_DENSE
    plan = _dense(inp, p, w.backward)
    rep = P.Report()
    for b in range(p.batch):
        for h in range(p.heads):
            q, k, v = f64(inp.q[b, h]), f64(inp.k[b, h]), f64(inp.v[b, h])
            o, lse = oracle.dense_forward_head(q, k, v)
            rep.add("O", plan.O[b, h].cpu().numpy(), o)
            rep.add("LSE", plan.LSE[b, h].cpu().numpy(), lse)
            if w.backward:
                dq, dk, dv = oracle.dense_backward_head(q, k, v, f64(inp.do[b, h]))
                rep.add("dQ", plan.dQ[b, h].cpu().numpy(), dq)
                rep.add("dK", plan.dK[b, h].cpu().numpy(), dk)
                rep.add("dV", plan.dV[b, h].cpu().numpy(), dv)
    print("DENSE " + json.dumps({"case": name, **rep.summary()}), flush=True)
    P.assert_float_parity(rep, bf16=w.dtype == "bf16")
    # the sparse path with all NB blocks kept walks the same blocks in the same order
    inp.k_per_head = np.full(p.heads, p.n_blocks, dtype=np.int32)
    run = P.run_gpu(inp)
    names = ("O", "LSE") + (("dQ", "dK", "dV") if w.backward else ())
    for n in names:
        assert torch.equal(getattr(plan, n), getattr(run.plan, n)), f"{n}: dense and keep-all sparse differ"


def test_dense_full_57k():
    """Full attention at 57,600 tokens (24-head, d = 128 layer; three heads run): O, LSE and dQ on
    sampled rows, dK and dV on two blocks of one head against the oracle, and on every head the
    column sums that hold at any size (dV rows add up to the dO rows, dK rows to zero)."""
    w = synth.workload(3)
    inp = synth.generate(w, heads=[0, 11, 23])
    p = P.problem_of(w, heads=3)
    plan = _dense(inp, p, True)
    groups = [0, 449, 899]
    rows = np.concatenate([np.arange(g * 64, (g + 1) * 64) for g in groups])
    rep, sums = P.Report(), P.Report()
    O, L, dQ, dK, dV = (getattr(plan, n)[0].cpu().numpy() for n in ("O", "LSE", "dQ", "dK", "dV"))
    assert all(np.isfinite(x).all() for x in (O, L, dQ, dK, dV))
    for h in range(3):
        q, k, v, do = (f64(getattr(inp, n)[0, h]) for n in ("q", "k", "v", "do"))
        o, lse = oracle.dense_rows(q[rows], k, v)
        rep.add("O", O[h][rows], o)
        rep.add("LSE", L[h][rows], lse)
        rep.add("dQ", dQ[h][rows], oracle.dense_dq_rows(q, k, v, do, rows))
        sums.add("sum_dV", dV[h].astype(np.float64).sum(axis=0), do.sum(axis=0))
        # zero reference: scale by what the sum is made of (N rows of dK with independent rounding)
        kscale = np.sqrt(k.shape[0]) * np.sqrt((dK[h].astype(np.float64) ** 2).sum(axis=1).mean())
        assert np.linalg.norm(dK[h].astype(np.float64).sum(axis=0)) <= P.BF16_REL_L2 * kscale
    print(f"CASE full_57k dK/dV blocks of head 0", flush=True)
    q, k, v, do = (f64(getattr(inp, n)[0, 0]) for n in ("q", "k", "v", "do"))
    for j, (rk, rv) in oracle.dense_dkdv_blocks(q, k, v, do, [0, p.n_blocks - 1]).items():
        rep.add("dK", dK[0][j * 64:(j + 1) * 64], rk)
        rep.add("dV", dV[0][j * 64:(j + 1) * 64], rv)
    print("DENSE " + json.dumps({"case": "full_57k", **rep.summary(), **sums.summary()}), flush=True)
    P.assert_float_parity(rep, bf16=True)
    assert sums.summary()["sum_dV"]["rel_l2"] <= P.BF16_REL_L2
