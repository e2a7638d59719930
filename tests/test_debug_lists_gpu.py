"""The debug build of the library (libdsa_debug.so, DSA_DEBUG): every attention call checks its kept-block
lists and reverse index on the device before launching anything.

Valid lists (written by the selection of the release library) give the release results bit for bit; each kind
of malformed list -- an id out of range, a repeated id, a reverse-list id out of range, a decreasing rev_ptr,
a varlen count out of range -- is rejected with DSA_ERR_BAD_LIST, a message on stderr, and no output
touched.  The checks only read list positions the layout defines, so the corrupt lists never reach a kernel
that would use their values as addresses.
"""
from __future__ import annotations

import os

import pytest
import torch

import synth
import dynamic_sparse_attention_qk_amd as dsa
from synth.device import problem_of, to_device

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(dsa.__file__), "libdsa_debug.so")


@pytest.fixture(scope="module")
def run():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DEBUG_LIB):
        pytest.skip("libdsa_debug.so is missing (python -m dynamic_sparse_attention_qk_amd.build)")
    dsa.library()
    w = synth.Workload("debug_lists", 4702, 1, 2, 128, (4, 16, 16), 8, 3.0, 32, 64, k=4)
    inp = synth.generate(w)
    p = problem_of(w)
    kph = [int(x) for x in inp.k_per_head]
    dev = {n: to_device(getattr(inp, n)) for n in ("q", "k", "v", "do", "w")}
    plan = dsa.SparseAttentionPlan(p, kph, reuse_v=False)
    plan.step(dev["q"], dev["k"], dev["v"], dev["w"], dev["w"], dev["do"])
    torch.cuda.synchronize()
    print(f"CASE debug lists N={w.seq_len} heads={w.heads} k={kph}", flush=True)
    return p, kph, dev, plan, dsa.load_library(DEBUG_LIB)


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def test_valid_lists_give_the_release_results(run, monkeypatch):
    p, kph, dev, plan, dbg = run
    monkeypatch.setattr(dsa, "_lib", dbg)
    O, LSE = torch.empty_like(plan.O), torch.empty_like(plan.LSE)
    dsa.sparse_attn_fwd(p, dev["q"], dev["k"], dev["v"], plan.idx, kph, O, LSE, plan.ws_fwd)
    dQ, dK, dV = (torch.empty_like(plan.dQ) for _ in range(3))
    dsa.sparse_attn_bwd(p, dev["q"], dev["k"], dev["v"], plan.O, dev["do"], plan.LSE, plan.idx, kph, plan.rev_ptr,
                        plan.rev_idx, dQ, dK, dV, plan.ws_bwd)
    torch.cuda.synchronize()
    for name, got, ref in (("O", O, plan.O), ("LSE", LSE, plan.LSE), ("dQ", dQ, plan.dQ), ("dK", dK, plan.dK),
                           ("dV", dV, plan.dV)):
        assert _same_bits(got, ref), name


CASES = ["idx_out_of_range", "idx_repeated", "rev_idx_out_of_range", "rev_ptr_decreasing", "varlen_count_zero"]


@pytest.mark.parametrize("case", CASES)
def test_malformed_list_is_rejected(run, monkeypatch, capfd, case):
    p, kph, dev, plan, dbg = run
    monkeypatch.setattr(dsa, "_lib", dbg)
    idx, rev_ptr, rev_idx = plan.idx.clone(), plan.rev_ptr.clone(), plan.rev_idx.clone()
    if case == "idx_out_of_range":
        idx[3] = p.n_blocks
    elif case == "idx_repeated":
        idx[5] = idx[4]
    elif case == "rev_idx_out_of_range":
        rev_idx[2] = p.n_groups
    elif case == "rev_ptr_decreasing":
        rev_ptr[0, 3] = rev_ptr[0, 2] - 1
    sentinel = float("nan")
    O = torch.full_like(plan.O, sentinel)
    LSE = torch.full_like(plan.LSE, sentinel)
    dQ, dK, dV = (torch.full_like(plan.dQ, sentinel) for _ in range(3))
    with pytest.raises(dsa.DsaError) as err:
        if case == "varlen_count_zero":
            cnt = torch.tensor(kph, dtype=torch.int32, device="cuda").view(1, -1, 1).repeat(p.batch, 1, p.n_groups)
            cnt[0, 1, 2] = 0  # counts are 1..k_h
            dsa.sparse_attn_fwd_varlen(p, dev["q"], dev["k"], dev["v"], idx, cnt, kph, O, LSE, plan.ws_fwd)
        elif case.startswith("idx"):
            dsa.sparse_attn_fwd(p, dev["q"], dev["k"], dev["v"], idx, kph, O, LSE, plan.ws_fwd)
        else:
            dsa.sparse_attn_bwd_dkdv(p, dev["q"], dev["k"], dev["v"], dev["do"], kph, rev_ptr, rev_idx, dK, dV,
                                     plan.ws_bwd)
    assert err.value.status == -9, err.value
    torch.cuda.synchronize()
    for name, t in (("O", O), ("LSE", LSE), ("dK", dK), ("dV", dV)):
        assert torch.isnan(t).all(), f"{name} was written although the call was rejected"
    assert "debug build" in capfd.readouterr().err
