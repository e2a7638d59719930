"""A seeded sweep of small problems through the whole path against the oracle (needs an MI355X).

Twenty-four problems drawn from a fixed seed vary everything the kernels branch on: head dim 64 / 128, group
64 / 128, predictor rank 8-64, batch 1-2, 1-3 heads, block counts that are ragged against the 64-wide
wavefront, a kept count per head anywhere in [1, NB], Morton or cube token order, materialised or streamed
scores, bf16 training steps and fp32 forwards.  Each is checked like the fixed small cases: predictor
outputs and scores to their tolerances, every kept list and reverse list exactly (on the GPU's own scores),
and every element of O, LSE, dQ, dK, dV at the literal bounds.
"""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import synth
import dynamic_sparse_attention_qk_amd as dsa
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.library()


def _draw(n: int = 24, seed: int = 20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        group = int(rng.choice([64, 128]))
        rank = int(rng.choice([8, 16, 32, 64]))
        heads = int(rng.integers(1, 4))
        batch = int(rng.integers(1, 3))
        fp32 = i % 6 == 5
        while True:
            grid = (int(rng.choice([2, 4])), int(rng.integers(3, 41)), int(rng.choice([8, 16, 24, 32, 48, 64])))
            n_tok = grid[0] * grid[1] * grid[2]
            if n_tok % group == 0 and n_tok // 64 >= 2:
                break
        nb = n_tok // 64
        kph = [int(rng.integers(1, nb + 1)) for _ in range(heads)]
        order = "cubes" if rng.random() < 0.5 else "morton"
        streamed = (not fp32) and rng.random() < 0.3
        name = (f"s{i}_d{d}_g{group}_r{rank}_b{batch}h{heads}_nb{nb}_k{'-'.join(map(str, kph))}_{order}"
                f"{'_f32fwd' if fp32 else ''}{'_streamed' if streamed else ''}")
        w = synth.Workload(name, 5000 + i, batch, heads, d, grid, int(rng.integers(2, 9)), 3.0, rank, group,
                           k=kph[0], dtype="f32" if fp32 else "bf16", backward=not fp32, order=order)
        out.append((name, w, kph, streamed))
    return out


CASES = _draw()


@pytest.mark.parametrize("name,w,kph,streamed", CASES, ids=[c[0] for c in CASES])
def test_sweep_parity(name, w, kph, streamed):
    print(f"CASE {name} N={w.seq_len}", flush=True)
    inp = synth.generate(w)
    inp.k_per_head = np.asarray(kph, dtype=np.int32)
    run = P.run_gpu(inp, materialise=not streamed, dump=streamed)
    rep = P.Report()
    P.check_predict_select(run, rep)
    P.check_forward(run, rep)
    if w.backward:
        P.check_backward(run, rep)
    print("PARITY " + json.dumps({"case": name, "score_err": rep.score_err, "idx_rows": rep.idx_rows,
                                  "errs": rep.summary()}), flush=True)
    P.assert_float_parity(rep, bf16=(w.dtype == "bf16"))
