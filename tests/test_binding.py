"""The Python binding's argument checks, without a GPU.

The C ABI takes bare device pointers, so the binding is where a tensor of the
wrong dtype or size, a host tensor, or a short k_per_head is caught: each such
mismatch must raise before anything reaches the library's compute calls.  The
checks run in the order dtype, size, layout, device, so host tensors can stand
in for device ones up to the last check.
"""
import pytest
import torch

import dynamic_sparse_attention_qk_amd as dsa

P = dsa.Problem(batch=1, heads=2, seq_len=1024, head_dim=64, rank=16, group=64)
KPH = [3, 5]


def _t(dtype, n):
    return torch.zeros(n, dtype=dtype)


def _fwd_args(**over):
    a = dict(Q=_t(torch.bfloat16, P.elems), K=_t(torch.bfloat16, P.elems), V=_t(torch.bfloat16, P.elems),
             idx=_t(torch.int32, P.list_len(KPH)), k_per_head=KPH, O=_t(torch.float32, P.elems),
             LSE=_t(torch.float32, P.rows), workspace=_t(torch.uint8, 16))
    a.update(over)
    return a


def test_sizes_of_the_problem():
    assert P.rows == 2 * 1024 and P.elems == 2 * 1024 * 64
    assert P.list_len(KPH) == 16 * 8


@pytest.mark.parametrize("name,bad", [
    ("Q", _t(torch.float32, P.elems)),          # fp32 for a bf16 problem
    ("V", _t(torch.float16, P.elems)),
    ("idx", _t(torch.int64, P.list_len(KPH))),
    ("O", _t(torch.bfloat16, P.elems)),
    ("LSE", _t(torch.float64, P.rows)),
])
def test_wrong_dtype_raises(name, bad):
    with pytest.raises(TypeError, match=name):
        dsa.sparse_attn_fwd(P, **_fwd_args(**{name: bad}))


@pytest.mark.parametrize("name,bad", [
    ("Q", _t(torch.bfloat16, P.elems - 1)),
    ("K", _t(torch.bfloat16, P.elems // 2)),
    ("idx", _t(torch.int32, P.list_len(KPH) - 1)),
    ("O", _t(torch.float32, P.elems - 64)),
    ("LSE", _t(torch.float32, P.rows - 1)),
])
def test_short_tensor_raises(name, bad):
    with pytest.raises(ValueError, match=name):
        dsa.sparse_attn_fwd(P, **_fwd_args(**{name: bad}))


def test_host_tensor_raises_on_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        dsa.sparse_attn_fwd(P, **_fwd_args())


def test_non_contiguous_raises():
    q = _t(torch.bfloat16, 2 * P.elems)[::2]
    with pytest.raises(ValueError, match="contiguous"):
        dsa.sparse_attn_fwd(P, **_fwd_args(Q=q))


def test_k_per_head_length_checked():
    with pytest.raises(ValueError, match="k_per_head"):
        dsa.sparse_attn_fwd(P, **_fwd_args(k_per_head=[3]))
    with pytest.raises(ValueError, match="k_per_head"):
        dsa.index_layout(P, [3, 5, 7])
    with pytest.raises(ValueError, match="k_per_head"):
        dsa.choose_path(P, [3])


def test_required_arguments():
    with pytest.raises(ValueError, match="idx"):
        dsa.sparse_attn_fwd(P, **_fwd_args(idx=None))
    with pytest.raises(ValueError, match="workspace"):
        dsa.sparse_attn_bwd_dq(P, _t(torch.bfloat16, P.elems), _t(torch.bfloat16, P.elems),
                               _t(torch.int32, P.list_len(KPH)), KPH, _t(torch.float32, P.elems), None)


def test_backward_and_selection_checks():
    n = P.list_len(KPH)
    grads = dict(dQ=_t(torch.float32, P.elems), dK=_t(torch.float32, P.elems), dV=_t(torch.float32, P.elems))
    qkvo = [_t(torch.bfloat16, P.elems) for _ in range(4)]
    with pytest.raises(TypeError, match="dK"):
        dsa.sparse_attn_bwd_dkdv(P, *qkvo, KPH, _t(torch.int32, 2 * 17), _t(torch.int32, n),
                                 _t(torch.float16, P.elems), grads["dV"], _t(torch.uint8, 16))
    with pytest.raises(ValueError, match="rev_ptr"):
        dsa.sparse_attn_bwd_dkdv(P, *qkvo, KPH, _t(torch.int32, 2 * 17 - 1), _t(torch.int32, n), grads["dK"],
                                 grads["dV"], _t(torch.uint8, 16))
    with pytest.raises(TypeError, match="dO"):
        dsa.sparse_attn_bwd_dkdv(P, *qkvo[:3], _t(torch.float32, P.elems), KPH, _t(torch.int32, 34),
                                 _t(torch.int32, n), grads["dK"], grads["dV"], _t(torch.uint8, 16))
    scores = _t(torch.float32, 2 * 16 * 16)
    with pytest.raises(ValueError, match="scores"):
        dsa.select_topk_blocks(P, scores[:-1], None, None, KPH, _t(torch.int32, n), _t(torch.int32, 34),
                               _t(torch.int32, n), _t(torch.uint8, 16))
    with pytest.raises(ValueError, match="rev_idx"):
        dsa.select_topk_blocks(P, scores, None, None, KPH, _t(torch.int32, n), _t(torch.int32, 34),
                               _t(torch.int32, n - 2), _t(torch.uint8, 16))
    with pytest.raises(TypeError, match="Wq"):
        dsa.predict_block_scores(P, _t(torch.bfloat16, P.elems), _t(torch.bfloat16, P.elems),
                                 _t(torch.float64, 2 * 64 * 16), _t(torch.float32, 2 * 64 * 16),
                                 _t(torch.float32, 2 * 16 * 16), _t(torch.float32, 2 * 16 * 16))


def test_fp32_problem_takes_fp32_inputs():
    p32 = dsa.Problem(batch=1, heads=2, seq_len=1024, head_dim=64, rank=16, group=64, dtype=dsa.DSA_F32)
    a = _fwd_args(Q=_t(torch.float32, P.elems), K=_t(torch.float32, P.elems), V=_t(torch.bfloat16, P.elems))
    with pytest.raises(TypeError, match="V"):
        dsa.sparse_attn_fwd(p32, **a)


def test_call_passes_arguments_then_the_stream(monkeypatch):
    seen = {}

    class FakeLib:
        def dsa_fake(self, *args):
            seen["args"] = args
            return 0

    monkeypatch.setattr(dsa, "library", lambda: FakeLib())
    monkeypatch.setattr(dsa, "_stream", lambda stream=None: ("stream", stream))
    a = dsa._Args(P)
    assert a.call("dsa_fake", 1, 2, stream="s") == 0
    assert seen["args"] == (1, 2, ("stream", "s"))
