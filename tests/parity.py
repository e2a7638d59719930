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
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch
from threadpoolctl import threadpool_limits

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

    def scores_head(self, b, h) -> np.ndarray:
        """The GPU's block scores of (b, h), [NG, NB] fp32, from host or copied from the device."""
        if "scores" in self.host:
            return self.host["scores"][b, h]
        return self.dev["scores"][b, h].cpu().numpy()

    def out_head(self, name, b, h) -> np.ndarray:
        """One (b, h) slice of a GPU output (O, LSE, dQ, dK, dV) on the host."""
        return getattr(self.plan, name)[b, h].cpu().numpy()

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
            keep_scores: bool = True, dump: bool = False, scores_on_device: bool = False) -> GpuRun:
    """predict -> select (host list check) -> fwd -> bwd on the GPU; copies the lists to host.

    The block scores (materialised, or dumped by a streamed selection) are copied to host too, unless
    ``scores_on_device``: then they stay in run.dev["scores"] and run.scores_head copies one head at a time.
    """
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
    src = plan.scores if materialise else dump_t
    if src is not None and scores_on_device:
        run.dev["scores"] = src
    elif src is not None and keep_scores:
        run.host["scores"] = src.cpu().numpy()
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
    for b in range(p.batch):
        for h in range(p.heads):
            if groups is not None and h not in groups:
                continue
            gl = None if groups is None else list(groups[h])
            q, k, v = f64(inp.q[b, h]), f64(inp.k[b, h]), f64(inp.v[b, h])
            o_ref, l_ref = oracle.forward_head(q, k, v, run.idx_rows(b, h), p.group, groups=gl)
            O, L = run.out_head("O", b, h), run.out_head("LSE", b, h)
            if gl is None:
                rep.add("O", O, o_ref)
                rep.add("LSE", L, l_ref)
            else:
                rows = np.concatenate([np.arange(g * p.group, (g + 1) * p.group) for g in gl])
                rep.add("O", O[rows], o_ref[rows])
                rep.add("LSE", L[rows], l_ref[rows])


def check_backward(run: GpuRun, rep: Report, groups: Optional[Dict[int, Sequence[int]]] = None,
                   blocks: Optional[Dict[int, Sequence[int]]] = None) -> None:
    inp, p = run.inp, run.plan.p
    G = p.group
    for b in range(p.batch):
        for h in range(p.heads):
            if groups is not None and h not in groups and (blocks is None or h not in blocks):
                continue
            q, k, v, do = f64(inp.q[b, h]), f64(inp.k[b, h]), f64(inp.v[b, h]), f64(inp.do[b, h])
            idx = run.idx_rows(b, h)
            dQ, dK, dV = run.out_head("dQ", b, h), run.out_head("dK", b, h), run.out_head("dV", b, h)
            if groups is None:
                dq, dk, dv = oracle.backward_head(q, k, v, do, idx, G)
                rep.add("dQ", dQ, dq)
                rep.add("dK", dK, dk)
                rep.add("dV", dV, dv)
                kept = np.zeros(p.n_blocks, dtype=bool)
                kept[np.unique(idx)] = True
                for j in np.nonzero(~kept)[0]:
                    assert (dK[j * 64:(j + 1) * 64] == 0).all() and (dV[j * 64:(j + 1) * 64] == 0).all()
                continue
            if h in groups:
                for g, ref in oracle.dq_groups(q, k, v, do, idx, G, groups[h]).items():
                    rep.add("dQ", dQ[g * G:(g + 1) * G], ref)
            if blocks is not None and h in blocks:
                for j, (rk, rv) in oracle.dkdv_blocks(q, k, v, do, idx, G, blocks[h]).items():
                    rep.add("dK", dK[j * 64:(j + 1) * 64], rk)
                    rep.add("dV", dV[j * 64:(j + 1) * 64], rv)


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


# ------------------------------------------------------------------ whole-layer checks (threaded oracle)

def _pool_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def check_selection_full(run: GpuRun, rep: Report, heads: Optional[Sequence[int]] = None,
                         threads: Optional[int] = None) -> None:
    """Stages 1-3 on every row of the listed heads (all by default), each head whole: scores against the
    oracle's (per-row relative error), the oracle's top-k of the GPU's scores against the GPU's lists (bit
    for bit), and the GPU's reverse index against the oracle's.  Heads run in parallel threads."""
    inp, p = run.inp, run.plan.p
    todo = [(b, h) for b in range(p.batch) for h in (range(p.heads) if heads is None else heads)]

    def one(bh):
        b, h = bh
        q, k = f64(inp.q[b, h]), f64(inp.k[b, h])
        wt = inp.w[h].astype(np.float64)
        qhat, khat, s_ref = oracle.predict_head(q, k, wt, wt, p.group)
        del q, k
        np.testing.assert_allclose(run.host["qhat"][b, h], qhat, rtol=1e-4, atol=1e-4 * np.abs(qhat).max())
        np.testing.assert_allclose(run.host["khat"][b, h], khat, rtol=1e-4, atol=1e-4 * np.abs(khat).max())
        s_gpu = run.scores_head(b, h).astype(np.float64)
        err = row_rel_err(s_gpu, s_ref)
        assert err <= SCORE_TOL, f"score error {err} (b={b}, h={h})"
        kk = int(inp.k_per_head[h])
        gidx = run.idx_rows(b, h)
        want = oracle.select_rows(s_gpu, kk)
        bad = np.nonzero((gidx != want).any(axis=1))[0]
        assert bad.size == 0, f"kept blocks differ at b={b} h={h} rows {bad[:8].tolist()}"
        own = int(((oracle.select_rows(s_ref, kk) != want).any(axis=1)).sum())
        ptr, groups = oracle.reverse_index_csr(gidx, p.n_blocks)
        rp = run.host["rev_ptr"][b * p.heads + h]
        base = int(run.plan.row_base[b * p.heads + h])
        assert np.array_equal(rp, ptr), f"reverse pointers differ at b={b} h={h}"
        assert np.array_equal(run.host["rev_idx"][base:base + groups.size], groups), f"reverse lists b={b} h={h}"
        return err, gidx.shape[0], own

    with ThreadPoolExecutor(threads or min(8, _pool_threads())) as ex:
        for err, rows, own in ex.map(one, todo):
            rep.score_err = max(rep.score_err, err)
            rep.idx_rows += rows
            rep.idx_own_mismatch += own


def _oracle_head(q, k, v, do, idx, group, threads):
    """O, LSE (and dQ, dK, dV when do is given) of one (b, h) by the oracle's per-group functions, the groups
    cut into contiguous chunks, one per thread; each thread sums its own dK, dV, added in chunk order."""
    n, d = q.shape
    ng = n // group
    o, lse = np.empty((n, d)), np.empty(n)
    dq = np.empty((n, d)) if do is not None else None

    def work(gs):
        dk = np.zeros_like(k) if do is not None else None
        dv = np.zeros_like(v) if do is not None else None
        for g in gs:
            rows = slice(g * group, (g + 1) * group)
            keys = oracle.kept_keys(idx[g])
            if do is None:
                o[rows], lse[rows], _ = oracle.group_forward(q[rows], k, v, keys)
                continue
            dq[rows], dk_p, dv_p, o[rows], lse[rows] = oracle.group_backward(q[rows], k, v, do[rows], keys)
            dk[keys] += dk_p
            dv[keys] += dv_p
        return dk, dv

    chunks = [c for c in np.array_split(np.arange(ng), threads) if c.size]
    with threadpool_limits(1), ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(work, chunks))
    if do is None:
        return o, lse, None, None, None
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    for pk, pv in parts:
        dk += pk
        dv += pv
    return o, lse, dq, dk, dv


def check_attention_full(run: GpuRun, rep: Report, heads: Optional[Sequence[int]] = None,
                         threads: Optional[int] = None) -> None:
    """O and LSE (and dQ, dK, dV for a training workload) of the listed heads (all by default), every
    element, against the oracle run with the GPU's lists; keys no group kept must get exactly zero dK, dV."""
    inp, p = run.inp, run.plan.p
    backward = hasattr(run.plan, "dQ")
    for b in range(p.batch):
        for h in (range(p.heads) if heads is None else heads):
            q, k, v = f64(inp.q[b, h]), f64(inp.k[b, h]), f64(inp.v[b, h])
            do = f64(inp.do[b, h]) if backward else None
            idx = run.idx_rows(b, h)
            o, lse, dq, dk, dv = _oracle_head(q, k, v, do, idx, p.group, threads or _pool_threads())
            rep.add("O", run.out_head("O", b, h), o)
            rep.add("LSE", run.out_head("LSE", b, h), lse)
            if backward:
                gdk, gdv = run.out_head("dK", b, h), run.out_head("dV", b, h)
                rep.add("dQ", run.out_head("dQ", b, h), dq)
                rep.add("dK", gdk, dk)
                rep.add("dV", gdv, dv)
                kept = np.zeros(p.n_blocks, dtype=bool)
                kept[np.unique(idx)] = True
                for j in np.nonzero(~kept)[0]:
                    assert (gdk[j * 64:(j + 1) * 64] == 0).all() and (gdv[j * 64:(j + 1) * 64] == 0).all()


def dkdv_block_threaded(q, k, v, do, idx, group, j, groups, threads=None):
    """dK, dV rows of block j: the oracle's per-group parts over its reverse list ``groups``, spread over
    threads (contiguous chunks, each summed in list order, chunks added in order)."""
    chunks = [c for c in np.array_split(np.asarray(groups), threads or _pool_threads()) if c.size]

    def work(gs):
        dk, dv = np.zeros((64, k.shape[1])), np.zeros((64, v.shape[1]))
        for g in gs:
            pk, pv = oracle.dkdv_block_part(q, k, v, do, idx[int(g)], group, int(g), j)
            dk += pk
            dv += pv
        return dk, dv

    with threadpool_limits(1), ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(work, chunks))
    dk, dv = np.zeros((64, k.shape[1])), np.zeros((64, v.shape[1]))
    for pk, pv in parts:
        dk += pk
        dv += pv
    return dk, dv
