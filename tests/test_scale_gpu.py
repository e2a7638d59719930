"""Input magnitudes far from 1: the fp16 copies are scaled per (b, h) slice and the results scaled back.

Every case multiplies stored bf16 inputs by exact powers of two (dO as small as training gradients are,
V and Q/K beyond fp16's range or deep in its subnormals) and compares the GPU with the float64 oracle run
on the same scaled inputs.  Each output is divided by the exact factor its true value carries (O by the
V factor, dV by the dO factor, dK by dO*V*Q, dQ by dO*V*K; LSE is unchanged when Q*K is), which turns the
literal bounds into the bounds of the unscaled problem: rel-L2 <= 1e-2 and max-abs <= 2e-2.
"""
from __future__ import annotations

import json
import math

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


def _scaled(a: np.ndarray, e: int) -> np.ndarray:
    """bf16 bit patterns times 2^e (exact: only the exponent field changes for these magnitudes)."""
    x = synth.bf16_bits_to_f32(a).astype(np.float64) * math.ldexp(1.0, e)
    out = synth.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(out).astype(np.float64), x), "scaling was not exact"
    return out


CASES = [  # name, exponents (Q, K, V, dO)
    ("dO_x2^-20", (0, 0, 0, -20)),
    ("dO_x2^-24", (0, 0, 0, -24)),
    ("dO_x2^12", (0, 0, 0, 12)),
    ("dO_x2^16", (0, 0, 0, 16)),
    ("V_x2^-16", (0, 0, -16, 0)),
    ("V_x2^12", (0, 0, 12, 0)),
    ("Q_x2^12_K_x2^-12", (12, -12, 0, 0)),
    ("Q_x2^-12_K_x2^12", (-12, 12, 0, 0)),
    ("all_x2^-30_dO_x2^-40", (-8, 8, -30, -40)),
]


@pytest.mark.parametrize("name,ex", CASES, ids=[c[0] for c in CASES])
def test_scaled_inputs(name, ex):
    eq, ek, ev, eo = ex
    w = synth.Workload(f"scale_{name}", 4700, 1, 3, 128, (4, 16, 24), 8, 3.0, 32, 64, k=5)
    inp = synth.generate(w)
    inp.q, inp.k, inp.v, inp.do = _scaled(inp.q, eq), _scaled(inp.k, ek), _scaled(inp.v, ev), _scaled(inp.do, eo)
    run = P.run_gpu(inp)
    rep = P.Report()
    P.check_predict_select(run, rep)
    # the oracle on the scaled inputs, every element; each output divided by its exact factor
    factor = {"O": ev, "LSE": None, "dQ": eo + ev + ek, "dK": eo + ev + eq, "dV": eo}
    ref = P.Report()
    P.check_forward(run, ref)
    P.check_backward(run, ref)
    out = {}
    for n, e in ref.summary().items():
        f = 1.0 if factor[n] is None else math.ldexp(1.0, -factor[n])
        out[n] = {"rel_l2": e["rel_l2"], "max_abs": e["max_abs"] * f, "max_ref": e["max_ref"] * f}
    print("SCALE " + json.dumps({"case": name, "exponents_QKVdO": ex, "errs_unscaled": out}), flush=True)
    bad = {n: e for n, e in out.items() if not (e["rel_l2"] <= P.BF16_REL_L2 and e["max_abs"] <= P.BF16_MAX_ABS)}
    assert not bad, f"outside tolerance: {bad}"


def test_reused_v_copy_gives_the_same_bits():
    """The backward reusing the forward's scaled copy of V gives bit-identical gradients."""
    w = synth.Workload("reuse_v", 4701, 1, 3, 128, (4, 16, 24), 8, 3.0, 32, 64, k=6)
    inp = synth.generate(w)
    inp.v = _scaled(inp.v, -9)
    inp.do = _scaled(inp.do, -22)
    p = P.problem_of(w)
    dev = {n: P.to_device(getattr(inp, n)) for n in ("q", "k", "v", "do", "w")}
    outs = []
    for reuse in (False, True):
        plan = dsa.SparseAttentionPlan(p, inp.k_per_head, reuse_v=reuse)
        assert plan.reuse_v == reuse
        plan.step(dev["q"], dev["k"], dev["v"], dev["w"], dev["w"], dev["do"])
        plan.backward_stages(dev["q"], dev["k"], dev["v"], dev["do"])
        torch.cuda.synchronize()
        outs.append({n: getattr(plan, n).cpu().numpy() for n in ("O", "LSE", "dQ", "dK", "dV")})
    for n in outs[0]:
        np.testing.assert_array_equal(outs[0][n].view(np.uint32), outs[1][n].view(np.uint32), err_msg=n)
