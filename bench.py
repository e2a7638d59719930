"""Throughput of the DSV sparse-attention hot path on one MI355X.

One step = predict_block_scores -> select_topk_blocks -> sparse_attn_fwd ->
sparse_attn_bwd over one batch of seeded synthetic video latents (inputs
resident in HBM).  Default workload: 57,600 tokens (16x45x80 latent grid),
24 heads, d = 128, G = 64, 10% of 900 KV blocks kept (k = 90), bf16.

Prints one JSON line.  value = effective TFLOP/s of the step: the counted
kept-block attention FLOPs (forward 4*G*64*d per kept (group, block) pair,
backward 2.5x that) divided by the whole step's time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_F32_MFMA = 157.3e12
PEAK_HBM = 8.0e12       # bytes/s
METRIC = "sparse-attn fwd+bwd effective TFLOP/s + tokens/s at 57.6k tokens, 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="workload id 1..5 (3 is the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--split-kv", type=int, default=0,
                    help="also time the split-KV forward in this many parts plus the (O, LSE) merge")
    ap.add_argument("--dispatch-sweep", action="store_true",
                    help="also time dense attention against the sparse step over a sweep of keep fractions "
                         "(the dispatcher's break-even sparsity)")
    ap.add_argument("--coverage", type=float, default=0.0,
                    help="also time the step with selection by attention coverage (this fraction; the workload's "
                         "k as each row's cap) and per-row counts")
    ap.add_argument("--pooled", choices=["max", "lse"], default=None,
                    help="also time the predictor variant that pools token-level logits (and the step with it)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed")
    ap.add_argument("--predictor-grad", action="store_true",
                    help="also time the stage-1 predictor loss + gradient call on the same inputs")
    ap.add_argument("--cold-reps", type=int, default=-1,
                    help="repetitions of the cache-flushed protocol (median and min; -1: 20, or 5 at >= 256k "
                         "tokens; 0: off)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    return ap.parse_args()


def kept_pairs(w, kph) -> int:
    return int(w.batch * w.n_groups * int(np.sum(kph)))


def cpu_baseline(inp, target_s: float):
    """The float64 oracle, as it stands, on a bounded sample of the same workload:
    heads in order, each predicted and selected whole, then fwd(+bwd) group by
    group until about target_s seconds of CPU work."""
    import oracle
    from synth.device import f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info() if t.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = inp.workload
    G = w.group
    elapsed, flops, groups_done, heads_used = 0.0, 0.0, 0, 0
    for h in range(inp.q.shape[1]):
        if elapsed >= target_s:
            break
        heads_used += 1
        q, k, v = f64(inp.q[0, h]), f64(inp.k[0, h]), f64(inp.v[0, h])
        do = f64(inp.do[0, h]) if inp.do is not None else None
        wt = inp.w[h].astype(np.float64)
        t0 = time.perf_counter()
        _, _, s = oracle.predict_head(q, k, wt, wt, G)
        kk = int(inp.k_per_head[h])
        idx = np.stack([oracle.select_row(s[g], kk) for g in range(w.n_groups)])
        per_group_sel = (time.perf_counter() - t0) / w.n_groups
        for g in range(w.n_groups):
            if elapsed >= target_s:
                break
            rows = slice(g * G, (g + 1) * G)
            keys = oracle.kept_keys(idx[g])
            t1 = time.perf_counter()
            if do is not None:
                oracle.group_backward(q[rows], k, v, do[rows], keys)
            else:
                oracle.group_forward(q[rows], k, v, keys)
            elapsed += time.perf_counter() - t1 + per_group_sel
            flops += 4.0 * G * 64 * w.head_dim * kk * (3.5 if do is not None else 1.0)
            groups_done += 1
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{groups_done} query groups ({G} tokens each) over {heads_used} head(s): predict+select "
                       f"of each head (time pro-rated per group) and {'fwd+bwd' if inp.do is not None else 'fwd'} "
                       f"of each group, float64 numpy; {elapsed:.1f} s of CPU time"),
            "tokens_per_s": groups_done * G / elapsed}


# the device code of the attention kernels (launch.hpp holds host declarations only)
KERNEL_SOURCES = ("dynamic_sparse_attention_qk_amd/csrc/attn_fwd.hip", "dynamic_sparse_attention_qk_amd/csrc/attn_bwd.hip",
                  "dynamic_sparse_attention_qk_amd/csrc/common.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernels_bf16_57k_tokens_traffic.md")


def kernel_source_hash() -> str:
    """sha256 over the sources the attention kernels are compiled from; a stored
    traffic figure is used only while this still matches."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (lines 'TRAFFIC kernel=... workload=... source_sha256=...
    fetch_bytes=... write_bytes=...'), or None when absent or stale."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    cur = kernel_source_hash()
    for line in open(TRAFFIC_FILE):
        if not line.startswith("TRAFFIC "):
            continue
        kv = dict(item.split("=", 1) for item in line.split()[1:])
        if kv.get("kernel") == kernel and kv.get("workload") == workload and kv.get("source_sha256") == cur:
            return int(float(kv["fetch_bytes"]) + float(kv["write_bytes"]))
    return None


def time_split_kv(args, p, plan, Q, K, V, stream, fwd_ms, f_fwd, w):
    """Split-KV forward over args.split_kv parts of every kept list, then the (O, LSE) merge, timed with
    HIP events on the bench stream (same inputs and lists as the step)."""
    import torch
    import dynamic_sparse_attention_qk_amd as dsa
    n = args.split_kv
    O_part = torch.empty((n,) + tuple(plan.O.shape), dtype=torch.float32, device=plan.O.device)
    L_part = torch.empty((n,) + tuple(plan.LSE.shape), dtype=torch.float32, device=plan.O.device)
    O = torch.empty_like(plan.O)
    L = torch.empty_like(plan.LSE)
    split_ms, merge_ms = [], []
    for i in range(args.warmup + args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        dsa.sparse_attn_fwd_split(p, Q, K, V, plan.idx, plan.k_per_head, n, O_part, L_part, plan.ws_fwd, stream)
        e[1].record(stream)
        dsa.attn_merge(p, n, O_part, L_part, O, L, stream)
        e[2].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            split_ms.append(e[0].elapsed_time(e[1]))
            merge_ms.append(e[1].elapsed_time(e[2]))
    rows = w.batch * w.heads * w.seq_len
    merge_bytes = (n + 1) * rows * (w.head_dim + 1) * 4        # read every part's O and LSE, write O and LSE
    sm, mm = float(np.mean(split_ms)), float(np.mean(merge_ms))
    return {"parts": n, "fwd_split_ms": round(sm, 4), "merge_ms": round(mm, 4),
            "fwd_split_tflops": round(f_fwd / (sm / 1e3) / 1e12, 2), "unsplit_fwd_ms": round(fwd_ms, 4),
            "merge_hbm_gbs": round(merge_bytes / (mm / 1e3) / 1e9, 1), "merge_hbm_frac": round(
                merge_bytes / (mm / 1e3) / PEAK_HBM, 4)}


def time_predictor_grad(args, p, Q, K, Wt, stream, w):
    """dsa_predictor_loss_grad on the step's Q, K and predictor weights, timed with HIP events on the bench
    stream.  Algorithmic HBM bytes: Q and K read once (everything else is B H (NG + NB) (d + r) floats plus
    the NG x NB difference matrix, which the call writes once and reads three times)."""
    import torch
    import dynamic_sparse_attention_qk_amd as dsa
    loss = torch.empty(w.heads, dtype=torch.float32, device=Q.device)
    dWq, dWk = torch.empty_like(Wt), torch.empty_like(Wt)
    ws = torch.empty(dsa.workspace_bytes(p, None, dsa.DSA_WS_PRED_GRAD), dtype=torch.uint8, device=Q.device)
    ms = []
    for i in range(args.warmup + args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dsa.predictor_loss_grad(p, Q, K, Wt, Wt, loss, dWq, dWk, ws, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            ms.append(e0.elapsed_time(e1))
    elt = 2 if w.dtype == "bf16" else 4
    qk_bytes = 2 * w.batch * w.heads * w.seq_len * w.head_dim * elt
    e_bytes = 4 * w.batch * w.heads * w.n_groups * w.n_blocks * 4
    t = float(np.mean(ms))
    return {"ms": round(t, 4), "qk_read_gb": round(qk_bytes / 1e9, 4),
            "hbm_gbs_algorithmic": round(qk_bytes / (t / 1e3) / 1e9, 1),
            "hbm_frac_algorithmic": round(qk_bytes / (t / 1e3) / PEAK_HBM, 4),
            "hbm_gbs_with_diff_matrix": round((qk_bytes + e_bytes) / (t / 1e3) / 1e9, 1)}


def time_coverage(args, p, kph, Q, K, V, Wt, dO, stream, w):
    """The step with coverage selection: predict, select by coverage, forward and backward over rows of
    different lengths, each stage timed with HIP events on the bench stream."""
    import torch
    import dynamic_sparse_attention_qk_amd as dsa
    plan = dsa.SparseAttentionPlan(p, kph, materialise_scores=not w.streamed, backward=dO is not None,
                                   coverage=args.coverage)
    plan.idx.zero_()
    plan.rev_idx.zero_()
    plan.predict(Q, K, Wt, Wt, stream)
    plan.select(stream)
    torch.cuda.synchronize()
    cnt = plan.cnt.cpu().numpy()
    assert cnt.min() >= 1 and cnt.max() <= max(kph), "count out of range"
    names = ["predict", "select", "fwd"] + (["bwd"] if dO is not None else [])
    stages = {n: [] for n in names}
    for i in range(args.warmup + args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        ev[0].record(stream)
        plan.predict(Q, K, Wt, Wt, stream)
        ev[1].record(stream)
        plan.select(stream)
        ev[2].record(stream)
        plan.forward(Q, K, V, stream)
        ev[3].record(stream)
        if dO is not None:
            plan.backward(Q, K, V, dO, stream)
            ev[4].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            for j, n in enumerate(names):
                stages[n].append(ev[j].elapsed_time(ev[j + 1]))
    ms = {n: float(np.mean(v)) for n, v in stages.items()}
    pairs = int(cnt.sum())
    unit = 64 * w.group * w.head_dim
    flops = 4.0 * unit * pairs * (3.5 if dO is not None else 1.0)
    step = sum(ms.values())
    return {"coverage": args.coverage, "cap": max(kph), "mean_count": round(float(cnt.mean()), 3),
            "max_count": int(cnt.max()), "capped_rows": int((cnt == max(kph)).sum()), "kept_pairs": pairs,
            "stage_ms": {n: round(v, 4) for n, v in ms.items()}, "ms_per_step": round(step, 4),
            "tflops": round(flops / (step / 1e3) / 1e12, 2),
            "tokens_per_s": round(w.batch * w.seq_len / (step / 1e3), 1)}


def time_pooled(args, p, kph, Q, K, Wt, stream, w):
    """The pooled-logit predictor on the step's inputs, timed with HIP events on the bench stream, then the
    top-k selection on its scores.  Work: the N x N low-rank product (2 N^2 r FLOP per head, fp16 MFMA)."""
    import torch
    import dynamic_sparse_attention_qk_amd as dsa
    pool = {"max": dsa.POOL_MAX, "lse": dsa.POOL_LSE}[args.pooled]
    plan = dsa.SparseAttentionPlan(p, kph, backward=False)
    ws = torch.empty(dsa.workspace_bytes(p, None, dsa.DSA_WS_PRED_POOLED), dtype=torch.uint8, device=Q.device)
    ms, sel = [], []
    for i in range(args.warmup + args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        dsa.predict_block_scores_pooled(p, Q, K, Wt, Wt, pool, plan.scores, ws, stream)
        ev[1].record(stream)
        plan.select(stream)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            ms.append(ev[0].elapsed_time(ev[1]))
            sel.append(ev[1].elapsed_time(ev[2]))
    t = float(np.mean(ms))
    flop = 2.0 * w.batch * w.heads * w.seq_len * w.seq_len * w.rank
    return {"pooling": args.pooled, "predict_ms": round(t, 4), "select_ms": round(float(np.mean(sel)), 4),
            "lowrank_tflops": round(flop / (t / 1e3) / 1e12, 2), "frac_of_fp16_peak": round(flop / (t / 1e3) / PEAK_BF16, 4)}


SWEEP_KEEP = (0.02, 0.05, 0.1, 0.2, 0.3, 0.5, 0.7, 0.8, 0.9, 0.95, 1.0)


def _crossing(xs, ys, level):
    """Largest x at which the piecewise-linear curve through (xs, ys) (xs ascending) is still below level."""
    best = None
    for (x0, y0), (x1, y1) in zip(zip(xs, ys), zip(xs[1:], ys[1:])):
        if y0 < level <= y1:
            best = x0 + (x1 - x0) * (level - y0) / (y1 - y0)
    if best is None:
        best = xs[-1] if ys[-1] < level else (xs[0] if ys[0] >= level else None)
    return best


def dispatch_sweep(args, w, stream):
    """Dense forward+backward against the sparse step (predict, select, forward, backward) at uniform keep
    fractions of the same layer shape, each timed with HIP events on the bench stream.  The break-even keep
    fraction f* is where the sparse step's time reaches the dense one's; the dispatcher's threshold on the
    sparsity is 1 - f*.  The same is reported for the forward alone."""
    import torch
    import synth
    import dynamic_sparse_attention_qk_amd as dsa
    from synth.device import problem_of, to_device

    wb = w.with_(backward=True)
    inp = synth.generate(wb)
    p = problem_of(wb)
    Q, K, V, dO = (to_device(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    Wt = to_device(inp.w)
    reps = max(args.steps // 4, 3)

    def timed(fns):
        """Mean ms of each of the callables in fns, run back to back, over reps passes after one warm-up."""
        out = [[] for _ in fns]
        for i in range(reps + 1):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
            ev[0].record(stream)
            for j, f in enumerate(fns):
                f()
                ev[j + 1].record(stream)
            torch.cuda.synchronize()
            if i:
                for j in range(len(fns)):
                    out[j].append(ev[j].elapsed_time(ev[j + 1]))
        return [float(np.mean(x)) for x in out]

    dense = dsa.DenseAttentionPlan(p)
    d_fwd, d_bwd = timed([lambda: dense.forward(Q, K, V, stream), lambda: dense.backward(Q, K, V, dO, stream)])
    del dense
    torch.cuda.empty_cache()
    unit = 64 * wb.group * wb.head_dim
    dense_flops = 14.0 * unit * wb.batch * wb.heads * wb.n_groups * wb.n_blocks
    rows = []
    for f in SWEEP_KEEP:
        k = synth.keep_to_k(f, wb.n_blocks)
        plan = dsa.SparseAttentionPlan(p, [k] * wb.heads, materialise_scores=not wb.streamed)
        plan.idx.zero_()
        plan.rev_idx.zero_()
        plan.predict(Q, K, Wt, Wt, stream)
        plan.select(stream)
        torch.cuda.synchronize()
        ids = plan.idx[: int(plan.row_base[-1])].cpu().numpy()
        assert ids.min() >= 0 and ids.max() < p.n_blocks, "kept-block list out of range"
        s_pred, s_fwd, s_bwd = timed([lambda: (plan.predict(Q, K, Wt, Wt, stream), plan.select(stream)),
                                      lambda: plan.forward(Q, K, V, stream),
                                      lambda: plan.backward(Q, K, V, dO, stream)])
        rows.append({"keep": f, "k": k, "predict_select_ms": round(s_pred, 4), "fwd_ms": round(s_fwd, 4),
                     "bwd_ms": round(s_bwd, 4), "step_ms": round(s_pred + s_fwd + s_bwd, 4),
                     "fwd_only_ms": round(s_pred + s_fwd, 4)})
        del plan
        torch.cuda.empty_cache()
    keeps = [r["k"] / wb.n_blocks for r in rows]
    f_step = _crossing(keeps, [r["step_ms"] for r in rows], d_fwd + d_bwd)
    f_fwd = _crossing(keeps, [r["fwd_only_ms"] for r in rows], d_fwd)
    return {"workload": wb.name, "seq_len": wb.seq_len, "heads": wb.heads, "head_dim": wb.head_dim,
            "group": wb.group, "dense_fwd_ms": round(d_fwd, 4), "dense_bwd_ms": round(d_bwd, 4),
            "dense_fwd_bwd_tflops": round(dense_flops / ((d_fwd + d_bwd) / 1e3) / 1e12, 2),
            "dense_fwd_tflops": round(dense_flops * 4 / 14 / (d_fwd / 1e3) / 1e12, 2),
            "sparse": rows,
            "break_even_keep_step": None if f_step is None else round(f_step, 4),
            "min_sparsity_step": None if f_step is None else round(1 - f_step, 4),
            "break_even_keep_fwd": None if f_fwd is None else round(f_fwd, 4),
            "min_sparsity_fwd": None if f_fwd is None else round(1 - f_fwd, 4)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import dynamic_sparse_attention_qk_amd as dsa
    from synth.device import problem_of, to_device

    w = synth.workload(args.workload)
    t0 = time.time()
    inp = synth.generate(w)
    print(f"# generated {w.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)          # every launch and every event of the step is on this stream
    if args.copy_probe_mib:
        # one elementwise kernel that reads n bytes and writes n bytes (a copy with
        # the bits inverted; a same-type copy_ would go to the DMA engines and
        # never show in the shader counters): the reference point that scales the
        # FETCH_SIZE / WRITE_SIZE counters of a --pmc run to bytes
        n = args.copy_probe_mib << 20
        src = torch.full((n // 4,), 7, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    p = problem_of(w)
    kph = [int(x) for x in inp.k_per_head]
    backward = w.backward
    plan = dsa.SparseAttentionPlan(p, kph, materialise_scores=not w.streamed, backward=backward)
    plan.idx.zero_()
    plan.rev_idx.zero_()
    Q, K, V = (to_device(getattr(inp, n)) for n in ("q", "k", "v"))
    Wt = to_device(inp.w)
    dO = to_device(inp.do) if backward else None
    torch.cuda.synchronize()

    names = ["predict", "select", "fwd"] + (["bwd_pre", "bwd_dkdv", "bwd_dq"] if backward else [])

    def step(marks=None):
        """One pass of the hot path, stage by stage (the backward as its three
        single-kernel stages, the same launches sparse_attn_bwd makes)."""
        rec = (lambda i: marks[i].record(stream)) if marks is not None else (lambda i: None)
        rec(0)
        plan.predict(Q, K, Wt, Wt, stream)
        rec(1)
        plan.select(stream)
        rec(2)
        plan.forward(Q, K, V, stream)
        rec(3)
        if backward:
            # the forward wrote its scaled fp16 copy of V into the backward's workspace (plan.reuse_v)
            dsa.sparse_attn_bwd_preprocess(p, Q, K, V, plan.O, dO, plan.LSE, plan.ws_bwd, stream,
                                           flags=dsa.BWD_V_FROM_FORWARD if plan.reuse_v else 0)
            rec(4)
            dsa.sparse_attn_bwd_dkdv(p, Q, K, V, dO, kph, plan.rev_ptr, plan.rev_idx, plan.dK, plan.dV, plan.ws_bwd,
                                     stream)
            rec(5)
            dsa.sparse_attn_bwd_dq(p, Q, dO, plan.idx, kph, plan.dQ, plan.ws_bwd, stream)
            rec(6)

    # first pass checked on the host: every kept-block id in range before the attention kernels read them
    plan.predict(Q, K, Wt, Wt, stream)
    plan.select(stream)
    torch.cuda.synchronize()
    idx_host = plan.idx[: int(plan.row_base[-1])].cpu().numpy()
    assert idx_host.min() >= 0 and idx_host.max() < p.n_blocks, "kept-block list out of range"
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(marks[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    # per-kernel durations from the events recorded between the launches of the timed steps
    stage_ms = {n: float(np.mean([m[i].elapsed_time(m[i + 1]) for m in marks])) for i, n in enumerate(names)}

    # cache-flushed protocol: before each repetition a 512 MiB write (twice the 256 MiB MALL, far above the
    # 32 MiB of L2) evicts what the previous step left in the caches; each repetition is timed alone and the
    # median and min are reported beside the K-step mean above
    cold = None
    reps = args.cold_reps if args.cold_reps >= 0 else (5 if w.seq_len >= 262144 else 20)
    if reps > 0:
        flush = torch.empty(512 << 18, dtype=torch.int32, device=dev)
        cmarks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(reps)]
        for r in range(reps):
            with torch.cuda.stream(stream):
                flush.fill_(r)
            step(cmarks[r])
        torch.cuda.synchronize()
        del flush
        per_rep = [m[0].elapsed_time(m[-1]) for m in cmarks]
        cold = {"reps": reps, "flush_mib": 512, "ms_per_step_median": float(np.median(per_rep)),
                "ms_per_step_min": float(np.min(per_rep)),
                "stage_ms_median": {n: round(float(np.median([m[i].elapsed_time(m[i + 1]) for m in cmarks])), 4)
                                    for i, n in enumerate(names)}}

    pairs = kept_pairs(w, kph)
    unit = 64 * w.group * w.head_dim            # G x Bk x d per kept (group, block) pair
    f_fwd = 4.0 * unit * pairs
    f_bwd = 2.5 * f_fwd if backward else 0.0
    step_s = ms_step / 1e3
    tflops = (f_fwd + f_bwd) / step_s / 1e12
    attn_ms = stage_ms["fwd"] + sum(stage_ms.get(n, 0.0) for n in ("bwd_pre", "bwd_dkdv", "bwd_dq"))
    kernel_flops = {"fwd": 4.0 * unit * pairs, "bwd_dkdv": 8.0 * unit * pairs, "bwd_dq": 6.0 * unit * pairs}
    kernel_names = {"fwd": "attn_fwd_bf16_kernel", "bwd_dkdv": "bwd_dkdv_kernel", "bwd_dq": "bwd_dq_kernel"}
    cand = [n for n in ("fwd", "bwd_dkdv", "bwd_dq") if n in stage_ms]
    dom = max(cand, key=lambda n: stage_ms[n])
    dom_tflops = kernel_flops[dom] / (stage_ms[dom] / 1e3) / 1e12
    peak = PEAK_BF16 if w.dtype == "bf16" else PEAK_F32_MFMA
    elt = 2 if w.dtype == "bf16" else 4
    sel_bytes = (w.batch * w.heads * w.n_groups * w.n_blocks * 4 if not w.streamed else 0) + \
        2 * 4 * pairs + w.batch * w.heads * (w.n_blocks + 1) * 4
    pred_bytes = 2 * w.batch * w.heads * w.seq_len * w.head_dim * elt + \
        (w.batch * w.heads * w.n_groups * w.n_blocks * 4 if not w.streamed else 0)
    traffic = stored_traffic(kernel_names[dom], w.name) if w.dtype == "bf16" else None
    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Voronoi-clustered video latents, Morton token order)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "head_dim": w.head_dim, "rank": w.rank, "group": w.group, "block": 64,
                   "k_per_head": kph if len(set(kph)) > 1 else kph[0], "backward": backward,
                   "scores": "streamed" if w.streamed else "materialised"},
        "tokens_per_s": round(w.batch * w.seq_len / step_s, 1),
        "attn_fwd_bwd_tflops": round((f_fwd + f_bwd) / (attn_ms / 1e3) / 1e12, 3),
        "counted_tflop_per_step": round((f_fwd + f_bwd) / 1e12, 4),
        "stage_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "predict_hbm_gbs": round(pred_bytes / (stage_ms["predict"] / 1e3) / 1e9, 1),
        # the HBM-bound stages against 8 TB/s: predict reads Q and K once and writes the scores; select reads
        # the scores and writes the kept-block list and its reverse index (plus rev_ptr)
        "hbm_stages": {
            "predict": {"bytes": pred_bytes, "gbs": round(pred_bytes / (stage_ms["predict"] / 1e3) / 1e9, 1),
                        "frac": round(pred_bytes / (stage_ms["predict"] / 1e3) / PEAK_HBM, 4)},
            "select": {"bytes": sel_bytes, "gbs": round(sel_bytes / (stage_ms["select"] / 1e3) / 1e9, 1),
                       "frac": round(sel_bytes / (stage_ms["select"] / 1e3) / PEAK_HBM, 4)}},
        "cold_cache": None if cold is None else {
            "reps": cold["reps"], "flush_mib": cold["flush_mib"],
            "ms_per_step_median": round(cold["ms_per_step_median"], 4),
            "ms_per_step_min": round(cold["ms_per_step_min"], 4),
            "tflops_median": round((f_fwd + f_bwd) / (cold["ms_per_step_median"] / 1e3) / 1e12, 3),
            "tflops_best": round((f_fwd + f_bwd) / (cold["ms_per_step_min"] / 1e3) / 1e12, 3),
            "stage_ms_median": cold["stage_ms_median"]},
        "roofline": {"kernel": kernel_names[dom], "bound": "mfma", "achieved": round(dom_tflops, 2),
                     "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(dom_tflops * 1e12 / peak, 4),
                     "traffic": traffic},
    }
    if args.split_kv:
        rec["split_kv"] = time_split_kv(args, p, plan, Q, K, V, stream, stage_ms["fwd"], f_fwd, w)
    if args.coverage:
        rec["coverage_select"] = time_coverage(args, p, kph, Q, K, V, Wt, dO, stream, w)
    if args.graph:
        # the same step captured once (after a warm-up on a side stream) and replayed: launch overhead removed
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            with torch.cuda.stream(side):
                plan.predict(Q, K, Wt, Wt)
                plan.select()
                plan.forward(Q, K, V)
                if backward:
                    plan.backward(Q, K, V, dO)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        rec["graph"] = {"ms_per_step": round(gms, 4), "tflops": round((f_fwd + f_bwd) / (gms / 1e3) / 1e12, 3),
                        "tokens_per_s": round(w.batch * w.seq_len / (gms / 1e3), 1)}
    if args.pooled:
        rec["pooled_predictor"] = time_pooled(args, p, kph, Q, K, Wt, stream, w)
    if args.predictor_grad:
        rec["predictor_grad"] = time_predictor_grad(args, p, Q, K, Wt, stream, w)
    if args.dispatch_sweep:
        del plan
        torch.cuda.empty_cache()
        rec["dispatch_sweep"] = dispatch_sweep(args, w, stream)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(inp, args.cpu_seconds)
        rec["cpu_baseline"] = cb
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
