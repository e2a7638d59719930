"""GPU-vs-oracle parity helpers: run the HIP hot path on seeded inputs and compare
each stage with the float64 oracle (test infrastructure; imports oracle/).

Protocol:
  1. block scores: per row, max_j |s - s_ref| / max_j |s_ref| <= 1e-3;
  2. kept blocks: the oracle's top-k applied to the GPU's own scores must equal
     the GPU's lists bit for bit (rows where the oracle's own scores would pick
     differently are counted, not failed: near-ties at the cut-off);
  3. reverse index: exactly the oracle's reverse index of the GPU's lists;
  4. attention outputs and gradients: the oracle run with the GPU's lists.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
import synth
import dynamic_sparse_attention_qk_amd as dsa
from synth.device import f64, problem_of, to_device  # noqa: F401 (re-exported for the tests)

SCORE_TOL = 1e-3
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 2e-2
F32_MAX_ABS = 1e-4


@dataclass
class GpuRun:
    inp: synth.Inputs
    plan: dsa.SparseAttentionPlan
    dev: Dict[str, torch.Tensor]
    host: Dict[str, np.ndarray] = field(default_factory=dict)

    def idx_rows(self, b, h) -> np.ndarray:
        rb = self.plan.row_base
        H = self.plan.p.heads
        s = int(rb[b * H + h])
        k = self.plan.k_per_head[h]
        return self.host["idx"][s:s + self.plan.p.n_groups * k].reshape(self.plan.p.n_groups, k)

    def rev_lists(self, b, h) -> List[np.ndarray]:
        p = self.plan.p
        rp = self.host["rev_ptr"][b * p.heads + h]
        base = int(self.plan.row_base[b * p.heads + h])
        ri = self.host["rev_idx"]
        return [ri[base + rp[j]: base + rp[j + 1]] for j in range(p.n_blocks)]


def validate_lists(run: GpuRun) -> None:
    """Host check that every kept-block list is in range, ascending and unique, and the
    reverse lists are consistent, before any kernel indexes memory with them."""
    p = run.plan.p
    for b in range(p.batch):
        for h in range(p.heads):
            rows = run.idx_rows(b, h)
            assert rows.min() >= 0 and rows.max() < p.n_blocks, "kept block id out of range"
            if rows.shape[1] > 1:
                assert (np.diff(rows, axis=1) > 0).all(), "kept-block rows not strictly ascending"
            rp = run.host["rev_ptr"][b * p.heads + h]
            assert rp[0] == 0 and rp[-1] == rows.size and (np.diff(rp) >= 0).all(), "bad reverse pointers"
    ri = run.host["rev_idx"][: int(run.plan.row_base[-1])]
    assert ri.min() >= 0 and ri.max() < p.n_groups, "reverse list group id out of range"


def run_gpu(inp: synth.Inputs, materialise: bool = True, backward: Optional[bool] = None,
            keep_scores: bool = True, dump: bool = False) -> GpuRun:
    """predict -> select (host list check) -> fwd -> bwd on the GPU; copies results to host."""
    w = inp.workload
    backward = w.backward if backward is None else backward
    p = problem_of(w, heads=inp.q.shape[1])
    plan = dsa.SparseAttentionPlan(p, inp.k_per_head, materialise_scores=materialise, backward=backward)
    plan.idx.zero_()
    plan.rev_idx.zero_()
    dev = {n: to_device(getattr(inp, n)) for n in ("q", "k", "v")}
    dev["w"] = to_device(inp.w)
    if backward:
        dev["do"] = to_device(inp.do)
    run = GpuRun(inp, plan, dev)
    plan.predict(dev["q"], dev["k"], dev["w"], dev["w"])
    dump_t = None
    if dump and not materialise:
        dump_t = torch.empty(p.batch, p.heads, p.n_groups, p.n_blocks, dtype=torch.float32, device="cuda")
    plan.select(scores_dump=dump_t)
    torch.cuda.synchronize()
    run.host["qhat"] = plan.qhat.cpu().numpy()
    run.host["khat"] = plan.khat.cpu().numpy()
    if materialise and keep_scores:
        run.host["scores"] = plan.scores.cpu().numpy()
    if dump_t is not None:
        run.host["scores"] = dump_t.cpu().numpy()
        del dump_t
    run.host["idx"] = plan.idx.cpu().numpy()
    run.host["rev_ptr"] = plan.rev_ptr.cpu().numpy()
    run.host["rev_idx"] = plan.rev_idx.cpu().numpy()
    validate_lists(run)
    plan.forward(dev["q"], dev["k"], dev["v"])
    if backward:
        plan.backward(dev["q"], dev["k"], dev["v"], dev["do"])
    torch.cuda.synchronize()
    return run


def rel_l2(x, ref) -> float:
    d = float(np.linalg.norm(ref))
    return float(np.linalg.norm(x - ref)) / (d if d > 0 else 1.0)


def row_rel_err(s, ref) -> float:
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((np.abs(s - ref).max(axis=-1) / den).max())


@dataclass
class Report:
    score_err: float = 0.0
    idx_rows: int = 0
    idx_own_mismatch: int = 0
    errs: Dict[str, Dict[str, float]] = field(default_factory=dict)

    def add(self, name, x, ref):
        e = self.errs.setdefault(name, {"rel_l2_num": 0.0, "rel_l2_den": 0.0, "max_abs": 0.0, "max_ref": 0.0})
        e["rel_l2_num"] += float(np.sum((x - ref) ** 2))
        e["rel_l2_den"] += float(np.sum(ref ** 2))
        e["max_abs"] = max(e["max_abs"], float(np.abs(x - ref).max()) if x.size else 0.0)
        e["max_ref"] = max(e["max_ref"], float(np.abs(ref).max()) if ref.size else 0.0)

    def summary(self) -> Dict[str, Dict[str, float]]:
        out = {}
        for n, e in self.errs.items():
            out[n] = {"rel_l2": math.sqrt(e["rel_l2_num"] / e["rel_l2_den"]) if e["rel_l2_den"] > 0 else 0.0,
                      "max_abs": e["max_abs"], "max_ref": e["max_ref"]}
        return out


def check_predict_select(run: GpuRun, rep: Report, heads: Optional[Sequence[int]] = None,
                         rows: Optional[Sequence[int]] = None, rev_blocks: Optional[Sequence[int]] = None) -> None:
    """Stages 1-3 for the listed heads (all by default) and rows (all by default).

    The reverse index is checked whole when ``rows`` is None, else on ``rev_blocks``.
    """
    inp, p = run.inp, run.plan.p
    for b in range(p.batch):
        for h in (range(p.heads) if heads is None else heads):
            q, k = f64(inp.q[b, h]), f64(inp.k[b, h])
            wt = inp.w[h].astype(np.float64)
            qhat, khat, s_ref = oracle.predict_head(q, k, wt, wt, p.group)
            np.testing.assert_allclose(run.host["qhat"][b, h], qhat, rtol=1e-4, atol=1e-4 * np.abs(qhat).max())
            np.testing.assert_allclose(run.host["khat"][b, h], khat, rtol=1e-4, atol=1e-4 * np.abs(khat).max())
            s_gpu = run.host["scores"][b, h].astype(np.float64)
            sel = range(p.n_groups) if rows is None else rows
            err = row_rel_err(s_gpu[list(sel)], s_ref[list(sel)])
            rep.score_err = max(rep.score_err, err)
            assert err <= SCORE_TOL, f"score error {err} (b={b}, h={h})"
            kk = int(inp.k_per_head[h])
            gidx = run.idx_rows(b, h)
            for g in sel:
                want = oracle.select_row(s_gpu[g], kk)
                assert np.array_equal(gidx[g], want), f"kept blocks differ at b={b} h={h} g={g}"
                rep.idx_rows += 1
                if not np.array_equal(oracle.select_row(s_ref[g], kk), want):
                    rep.idx_own_mismatch += 1
            rev = run.rev_lists(b, h)
            if rows is None:
                ref_rev = oracle.reverse_index(gidx, p.n_blocks)
                for j in range(p.n_blocks):
                    assert np.array_equal(rev[j], ref_rev[j]), f"reverse list differs at b={b} h={h} j={j}"
            else:
                for j in (rev_blocks or []):
                    assert np.array_equal(rev[j], oracle.reverse_list(gidx, j)), f"reverse list b={b} h={h} j={j}"


def check_forward(run: GpuRun, rep: Report, groups: Optional[Dict[int, Sequence[int]]] = None) -> None:
    """O and LSE vs the oracle with the GPU's lists; ``groups`` maps head -> sampled groups."""
    inp, p = run.inp, run.plan.p
    O = run.plan.O.cpu().numpy()
    L = run.plan.LSE.cpu().numpy()
    for b in range(p.batch):
        for h in range(p.heads):
            if groups is not None and h not in groups:
                continue
            gl = None if groups is None else list(groups[h])
            q, k, v = f64(inp.q[b, h]), f64(inp.k[b, h]), f64(inp.v[b, h])
            o_ref, l_ref = oracle.forward_head(q, k, v, run.idx_rows(b, h), p.group, groups=gl)
            if gl is None:
                rows = slice(None)
                rep.add("O", O[b, h], o_ref)
                rep.add("LSE", L[b, h], l_ref)
            else:
                rows = np.concatenate([np.arange(g * p.group, (g + 1) * p.group) for g in gl])
                rep.add("O", O[b, h][rows], o_ref[rows])
                rep.add("LSE", L[b, h][rows], l_ref[rows])


def check_backward(run: GpuRun, rep: Report, groups: Optional[Dict[int, Sequence[int]]] = None,
                   blocks: Optional[Dict[int, Sequence[int]]] = None) -> None:
    inp, p = run.inp, run.plan.p
    dQ = run.plan.dQ.cpu().numpy()
    dK = run.plan.dK.cpu().numpy()
    dV = run.plan.dV.cpu().numpy()
    G = p.group
    for b in range(p.batch):
        for h in range(p.heads):
            q, k, v, do = f64(inp.q[b, h]), f64(inp.k[b, h]), f64(inp.v[b, h]), f64(inp.do[b, h])
            idx = run.idx_rows(b, h)
            if groups is None:
                dq, dk, dv = oracle.backward_head(q, k, v, do, idx, G)
                rep.add("dQ", dQ[b, h], dq)
                rep.add("dK", dK[b, h], dk)
                rep.add("dV", dV[b, h], dv)
                kept = np.zeros(p.n_blocks, dtype=bool)
                kept[np.unique(idx)] = True
                for j in np.nonzero(~kept)[0]:
                    assert (dK[b, h, j * 64:(j + 1) * 64] == 0).all() and (dV[b, h, j * 64:(j + 1) * 64] == 0).all()
                continue
            if h in groups:
                for g, ref in oracle.dq_groups(q, k, v, do, idx, G, groups[h]).items():
                    rep.add("dQ", dQ[b, h, g * G:(g + 1) * G], ref)
            if blocks is not None and h in blocks:
                for j, (rk, rv) in oracle.dkdv_blocks(q, k, v, do, idx, G, blocks[h]).items():
                    rep.add("dK", dK[b, h, j * 64:(j + 1) * 64], rk)
                    rep.add("dV", dV[b, h, j * 64:(j + 1) * 64], rv)


def assert_float_parity(rep: Report, bf16: bool, names=("O", "LSE", "dQ", "dK", "dV")) -> Dict:
    """Literal bounds: bf16 inputs -> rel-L2 <= 1e-2 and max-abs <= 2e-2; fp32 -> max-abs <= 1e-4."""
    s = rep.summary()
    bad = []
    for n in names:
        if n not in s:
            continue
        e = s[n]
        if bf16:
            if not (e["rel_l2"] <= BF16_REL_L2 and e["max_abs"] <= BF16_MAX_ABS):
                bad.append((n, e))
        elif not e["max_abs"] <= F32_MAX_ABS:
            bad.append((n, e))
    assert not bad, f"outside tolerance: {bad}"
    return s
