"""Split-KV forward (partial attention states over parts of each kept list) and the
(O, LSE) merge, on the GPU, against the float64 oracle's partial states and its
unsplit forward.  The partials are compared part by part; parts left empty (more
parts than kept blocks) must be exactly O = 0, LSE = -inf."""
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


def _wl(grid, heads, d, group, k, rank, seed=91):
    return synth.Workload(f"split_{grid}_{heads}_{d}_{group}", seed, 1, heads, d, grid, 8, 3.0, rank, group, k=k,
                          backward=False)


CASES = [
    # name, workload, per-head k override, part counts (some exceed k: empty parts)
    ("cfg1_fp32", synth.workload(1), None, (1, 2, 3, 6)),
    ("d128_g64", _wl((4, 20, 24), 2, 128, 64, k=7, rank=32), None, (1, 2, 3, 7, 9)),
    ("d64_g128", _wl((8, 16, 16), 2, 64, 128, k=6, rank=16), None, (2, 4)),
    ("d128_ragged_heads", _wl((4, 16, 32), 4, 128, 64, k=1, rank=64), [1, 3, 32, 9], (2, 5, 40)),
]


# Split vs unsplit on the GPU.  bf16 path: every part normalises its weights against its own running
# maximum before rounding them to fp16 (half an ulp, 2^-11 relative), so the two computations round
# differently: O may differ by about 2 x 2^-11 of max|O| and LSE (a log of sums of those weights) by
# about 2^-10; the bounds leave a 2x margin.  fp32 path: fp32 arithmetic throughout.
_SELF_O = {True: 2e-3, False: 1e-5}
_SELF_LSE = {True: 2e-3, False: 1e-4}


def _split(run, n):
    plan, dev, p = run.plan, run.dev, run.plan.p
    O_part = torch.empty((n,) + tuple(plan.O.shape), dtype=torch.float32, device="cuda")
    L_part = torch.empty((n,) + tuple(plan.LSE.shape), dtype=torch.float32, device="cuda")
    dsa.sparse_attn_fwd_split(p, dev["q"], dev["k"], dev["v"], plan.idx, plan.k_per_head, n, O_part, L_part,
                              plan.ws_fwd)
    O = torch.empty_like(plan.O)
    L = torch.empty_like(plan.LSE)
    dsa.attn_merge(p, n, O_part, L_part, O, L)
    torch.cuda.synchronize()
    return O_part.cpu().numpy(), L_part.cpu().numpy(), O.cpu().numpy(), L.cpu().numpy()


def _add_parts(rep, o, l, o_ref, l_ref):
    """Finite partial states into the report; empty ones (oracle LSE = -inf) must be exact."""
    empty = np.isneginf(l_ref)
    assert np.isneginf(l[empty]).all(), "an empty part must have LSE = -inf"
    assert (o[empty] == 0).all(), "an empty part must have O = 0"
    keep = ~empty
    rep.add("O_part", o[keep], o_ref[keep])
    rep.add("LSE_part", l[keep], l_ref[keep])
    return int(empty.sum())


@pytest.mark.parametrize("name,w,kph,splits", CASES, ids=[c[0] for c in CASES])
def test_split_kv_parity(name, w, kph, splits):
    print(f"CASE {name} N={w.seq_len} H={w.heads} d={w.head_dim} G={w.group} splits={splits}", flush=True)
    inp = synth.generate(w)
    if kph is not None:
        inp.k_per_head = np.asarray(kph, dtype=np.int32)
    run = P.run_gpu(inp, backward=False)
    p = run.plan.p
    bf16 = w.dtype == "bf16"
    O_plain, L_plain = run.plan.O.cpu().numpy(), run.plan.LSE.cpu().numpy()
    for n in splits:
        O_part, L_part, O_m, L_m = _split(run, n)
        rep_p, rep_m = P.Report(), P.Report()
        n_empty = 0
        for b in range(p.batch):
            for h in range(p.heads):
                q, k, v = f64(inp.q[b, h]), f64(inp.k[b, h]), f64(inp.v[b, h])
                idx = run.idx_rows(b, h)
                o_p, l_p = oracle.forward_split_head(q, k, v, idx, p.group, n)
                n_empty += _add_parts(rep_p, O_part[:, b, h], L_part[:, b, h], o_p, l_p)
                o_ref, l_ref = oracle.forward_head(q, k, v, idx, p.group)
                rep_m.add("O", O_m[b, h], o_ref)
                rep_m.add("LSE", L_m[b, h], l_ref)
        if n == 1:   # one part is the plain forward, launch for launch
            assert np.array_equal(O_part[0], O_plain) and np.array_equal(L_part[0], L_plain)
        # the merge of the GPU's own parts against its unsplit forward differs by rounding only
        assert np.abs(O_m - O_plain).max() <= _SELF_O[bf16] * np.abs(O_plain).max()
        assert np.abs(L_m - L_plain).max() <= _SELF_LSE[bf16]
        print("SPLIT " + json.dumps({"case": name, "n_split": n, "empty_rows": n_empty,
                                     "parts": rep_p.summary(), "merged": rep_m.summary()}), flush=True)
        P.assert_float_parity(rep_m, bf16=bf16, names=("O", "LSE"))
        sp = rep_p.summary()
        if bf16:
            assert sp["O_part"]["rel_l2"] <= P.BF16_REL_L2 and sp["O_part"]["max_abs"] <= P.BF16_MAX_ABS
            assert sp["LSE_part"]["rel_l2"] <= P.BF16_REL_L2 and sp["LSE_part"]["max_abs"] <= P.BF16_MAX_ABS
        else:
            assert sp["O_part"]["max_abs"] <= P.F32_MAX_ABS and sp["LSE_part"]["max_abs"] <= P.F32_MAX_ABS


def test_split_kv_full_57k():
    """The 57,600-token workload in 4 parts: merged vs the unsplit GPU forward on every row, partial states
    and the merge vs the oracle on sampled groups of three heads."""
    w = synth.workload(3).with_(backward=False)
    inp = synth.generate(w, heads=[0, 11, 23])
    run = P.run_gpu(inp, backward=False)
    p = run.plan.p
    n = 4
    O_part, L_part, O_m, L_m = _split(run, n)
    O_plain, L_plain = run.plan.O.cpu().numpy(), run.plan.LSE.cpu().numpy()
    assert np.abs(O_m - O_plain).max() <= _SELF_O[True] * np.abs(O_plain).max()
    assert np.abs(L_m - L_plain).max() <= _SELF_LSE[True]
    rep_p, rep_m = P.Report(), P.Report()
    groups = [0, 1, 449, 450, 898, 899]
    rows = np.concatenate([np.arange(g * p.group, (g + 1) * p.group) for g in groups])
    for h in range(p.heads):
        q, k, v = f64(inp.q[0, h]), f64(inp.k[0, h]), f64(inp.v[0, h])
        idx = run.idx_rows(0, h)
        o_p, l_p = oracle.forward_split_head(q, k, v, idx, p.group, n, groups=groups)
        _add_parts(rep_p, O_part[:, 0, h][:, rows], L_part[:, 0, h][:, rows], o_p[:, rows], l_p[:, rows])
        o_ref, l_ref = oracle.forward_head(q, k, v, idx, p.group, groups=groups)
        rep_m.add("O", O_m[0, h][rows], o_ref[rows])
        rep_m.add("LSE", L_m[0, h][rows], l_ref[rows])
    print("SPLIT " + json.dumps({"case": "full_57k", "n_split": n, "parts": rep_p.summary(),
                                 "merged": rep_m.summary()}), flush=True)
    P.assert_float_parity(rep_m, bf16=True, names=("O", "LSE"))
    sp = rep_p.summary()
    assert sp["O_part"]["rel_l2"] <= P.BF16_REL_L2 and sp["O_part"]["max_abs"] <= P.BF16_MAX_ABS
    assert sp["LSE_part"]["rel_l2"] <= P.BF16_REL_L2 and sp["LSE_part"]["max_abs"] <= P.BF16_MAX_ABS
