"""The C ABI without a GPU: the library loads, exports what include/dsa.h declares,
and host-side validation rejects bad arguments before anything is launched."""
import ctypes
import os
import re

import pytest

import dynamic_sparse_attention_qk_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            names += re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dsa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("dsa_predict_block_scores", "dsa_select_topk_blocks", "dsa_sparse_attn_fwd", "dsa_sparse_attn_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = dsa.library()
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(dsa.EXPORTED)
    assert "gfx950" in dsa.version()


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first


def _p(**kw):
    base = dict(batch=1, heads=2, seq_len=1024, head_dim=64, rank=16, group=64, block=64, dtype=dsa.DSA_BF16)
    base.update(kw)
    return dsa.Problem(**base)


def _fwd(p, kph, ptr=FAKE):
    lib = dsa.library()
    return lib.dsa_sparse_attn_fwd(ctypes.byref(p.c()), ptr, ptr, ptr, ptr, dsa._kph(kph), ptr, ptr, ptr, 1 << 40,
                                   None)


@pytest.mark.parametrize("kw,status", [
    (dict(seq_len=1000), -2),            # not a multiple of the block
    (dict(seq_len=64 * 3, group=128), -2),  # not a multiple of the group
    (dict(head_dim=96), -5),
    (dict(rank=12), -5),
    (dict(group=32), -5),
    (dict(block=32), -5),
    (dict(dtype=7), -3),
    (dict(heads=0), -2),
    (dict(heads=129), -5),
    (dict(seq_len=64 * 8193), -5),       # more than 8192 blocks
])
def test_bad_problem_rejected(kw, status):
    p = _p(**kw)
    assert _fwd(p, [1] * max(p.heads, 1)) == status


def test_bad_k_rejected():
    p = _p()
    assert _fwd(p, [0, 1]) == -2
    assert _fwd(p, [1, 17]) == -2      # k > NB = 16


def test_null_and_misaligned_pointers():
    lib = dsa.library()
    p = _p()
    kph = dsa._kph([4, 4])
    big = 1 << 40
    assert lib.dsa_sparse_attn_fwd(ctypes.byref(p.c()), None, FAKE, FAKE, FAKE, kph, FAKE, FAKE, FAKE, big, None) == -1
    bad = ctypes.c_void_p(0x100004)
    assert lib.dsa_sparse_attn_fwd(ctypes.byref(p.c()), FAKE, bad, FAKE, FAKE, kph, FAKE, FAKE, FAKE, big, None) == -4
    assert lib.dsa_sparse_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, kph, FAKE, FAKE, FAKE, big, None) == -1
    assert lib.dsa_sparse_attn_fwd(ctypes.byref(p.c()), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, big,
                                   None) == -1
    # bf16 forward needs the fp16 copy of V
    assert lib.dsa_sparse_attn_fwd(ctypes.byref(p.c()), FAKE, FAKE, FAKE, FAKE, kph, FAKE, FAKE, None, 0, None) == -6
    need = dsa.workspace_bytes(p, [4, 4], dsa.DSA_WS_FWD)
    assert need >= 2 * 1024 * 64 * 2
    assert lib.dsa_sparse_attn_fwd(ctypes.byref(p.c()), FAKE, FAKE, FAKE, FAKE, kph, FAKE, FAKE, FAKE, need - 1,
                                   None) == -6


def test_workspace_checks():
    lib = dsa.library()
    p = _p()
    kph = [4, 4]
    need = dsa.workspace_bytes(p, kph, dsa.DSA_WS_SELECT)
    # per-block counts [B*H, NB] + membership bitmaps [B*H, ceil(NG/32), NB] (NB = NG = 16 here)
    assert need >= 2 * 16 * 4 + 2 * 1 * 16 * 4
    assert dsa.workspace_bytes(p, kph, dsa.DSA_WS_BWD) >= 2 * 1024 * 4
    assert dsa.workspace_bytes(_p(seq_len=1000), kph, 0) == 0
    st = lib.dsa_select_topk_blocks(ctypes.byref(p.c()), FAKE, FAKE, FAKE, dsa._kph(kph), FAKE, FAKE, FAKE, None,
                                    FAKE, need - 1, None)
    assert st == -6
    st = lib.dsa_select_topk_blocks(ctypes.byref(p.c()), FAKE, FAKE, FAKE, dsa._kph(kph), FAKE, FAKE, FAKE, None,
                                    None, need, None)
    assert st == -6
    st = lib.dsa_sparse_attn_bwd(ctypes.byref(p.c()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dsa._kph(kph), FAKE,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == -6
    pf = _p(dtype=dsa.DSA_F32)
    st = lib.dsa_sparse_attn_bwd(ctypes.byref(pf.c()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dsa._kph(kph), FAKE,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == -3                      # backward is bf16-only


def test_index_layout_ragged():
    p = _p(batch=2, heads=3, seq_len=640)
    kph = [1, 5, 10]
    rb = dsa.index_layout(p, kph)
    ng = 10
    assert list(rb) == [0, ng * 1, ng * 6, ng * 16, ng * 17, ng * 22, ng * 32]
    with pytest.raises(dsa.DsaError):
        dsa.index_layout(p, [1, 5, 11])


def test_status_strings():
    for s in range(0, -10, -1):
        assert dsa.status_string(s) != "unknown status"
    assert dsa.status_string(5) == "unknown status"


def test_split_and_merge_validation():
    lib = dsa.library()
    p = _p()
    kph = dsa._kph([4, 4])
    big = 1 << 40
    pc = ctypes.byref(p.c())
    for n in (0, -1, dsa.MAX_SPLIT + 1):
        assert lib.dsa_sparse_attn_fwd_split(pc, FAKE, FAKE, FAKE, FAKE, kph, n, FAKE, FAKE, FAKE, big, None) == -1
        assert lib.dsa_attn_merge(pc, n, FAKE, FAKE, FAKE, FAKE, None) == -1
    bad = ctypes.c_void_p(0x100004)
    assert lib.dsa_sparse_attn_fwd_split(pc, FAKE, FAKE, FAKE, FAKE, kph, 2, None, FAKE, FAKE, big, None) == -1
    assert lib.dsa_sparse_attn_fwd_split(pc, FAKE, FAKE, FAKE, FAKE, kph, 2, FAKE, bad, FAKE, big, None) == -4
    assert lib.dsa_sparse_attn_fwd_split(pc, FAKE, FAKE, FAKE, FAKE, kph, 2, FAKE, FAKE, None, 0, None) == -6
    assert lib.dsa_sparse_attn_fwd_split(pc, FAKE, FAKE, FAKE, FAKE, dsa._kph([0, 4]), 2, FAKE, FAKE, FAKE, big,
                                         None) == -2
    assert lib.dsa_attn_merge(pc, 2, FAKE, FAKE, None, FAKE, None) == -1
    assert lib.dsa_attn_merge(pc, 2, FAKE, FAKE, FAKE, bad, None) == -4
    assert lib.dsa_attn_merge(ctypes.byref(_p(head_dim=96).c()), 2, FAKE, FAKE, FAKE, FAKE, None) == -5


def test_dense_calls_validation():
    lib = dsa.library()
    big = 1 << 40
    p = _p()
    pc = ctypes.byref(p.c())
    # forward: null, misaligned, missing workspace (bf16 needs one), bad problem
    assert lib.dsa_dense_attn_fwd(pc, None, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert lib.dsa_dense_attn_fwd(pc, FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None) == -1
    assert lib.dsa_dense_attn_fwd(pc, FAKE, ctypes.c_void_p(0x100004), FAKE, FAKE, FAKE, FAKE, big, None) == -4
    assert lib.dsa_dense_attn_fwd(pc, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -6
    need = dsa.workspace_bytes(p, None, dsa.DSA_WS_FWD)
    assert need == dsa.workspace_bytes(p, [3, 5], dsa.DSA_WS_FWD) > 0
    assert lib.dsa_dense_attn_fwd(pc, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == -6
    assert lib.dsa_dense_attn_fwd(ctypes.byref(_p(head_dim=96).c()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big,
                                  None) == -5
    assert lib.dsa_dense_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    # backward: bf16 only, nine tensors, DSA_WS_BWD
    args = [FAKE] * 9
    f32 = ctypes.byref(_p(dtype=dsa.DSA_F32).c())
    assert lib.dsa_dense_attn_bwd(f32, *args, FAKE, big, None) == -3
    for i in range(9):
        bad = list(args)
        bad[i] = None
        assert lib.dsa_dense_attn_bwd(pc, *bad, FAKE, big, None) == -1, i
        bad[i] = ctypes.c_void_p(0x100008)
        assert lib.dsa_dense_attn_bwd(pc, *bad, FAKE, big, None) == -4, i
    need = dsa.workspace_bytes(p, None, dsa.DSA_WS_BWD)
    assert need == dsa.workspace_bytes(p, [16, 16], dsa.DSA_WS_BWD) > 0
    assert lib.dsa_dense_attn_bwd(pc, *args, FAKE, need - 1, None) == -6
    assert lib.dsa_dense_attn_bwd(pc, *args, None, big, None) == -6
    # the selection workspace still needs the kept counts
    assert dsa.workspace_bytes(p, None, dsa.DSA_WS_SELECT) == 0


def _sparsity(kph, nb):
    return 1.0 - sum(kph) / (len(kph) * nb)


def test_default_threshold_matches_header():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    assert float(re.search(r"#define DSA_DEFAULT_MIN_SPARSITY ([0-9.]+)", text).group(1)) == dsa.DEFAULT_MIN_SPARSITY


def test_choose_path_rule():
    p = _p(heads=3)                    # NB = 16
    for kph in ([16, 16, 16], [15, 16, 16], [8, 8, 8], [1, 1, 1], [2, 16, 9], [14, 14, 14]):
        for thr in (0.0, 0.01, 0.1, 0.5, 0.9):
            want = dsa.PATH_SPARSE if _sparsity(kph, 16) > thr else dsa.PATH_DENSE
            assert dsa.choose_path(p, kph, thr) == want, (kph, thr)
    assert dsa.choose_path(p, [8, 8, 8], 0.5) == dsa.PATH_DENSE       # exactly at the threshold
    # the default threshold (any negative value, or NaN)
    lib = dsa.library()
    for kph in ([16, 16, 16], [15, 16, 16], [15, 15, 15], [14, 15, 15], [1, 1, 1]):   # sparsity 0 .. 0.94
        for thr in (-1.0, float("nan")):
            got = lib.dsa_choose_path(ctypes.byref(p.c()), dsa._kph(kph), thr, 0)
            assert got == (dsa.PATH_SPARSE if _sparsity(kph, 16) > dsa.DEFAULT_MIN_SPARSITY else dsa.PATH_DENSE)
    # invalid arguments
    assert lib.dsa_choose_path(ctypes.byref(p.c()), None, 0.1, 0) == -1
    assert lib.dsa_choose_path(None, dsa._kph([1, 1, 1]), 0.1, 0) == -1
    assert lib.dsa_choose_path(ctypes.byref(p.c()), dsa._kph([0, 1, 1]), 0.1, 0) == -2
    assert lib.dsa_choose_path(ctypes.byref(p.c()), dsa._kph([1, 17, 1]), 0.1, 0) == -2
    with pytest.raises(dsa.DsaError):
        dsa.choose_path(_p(head_dim=96), [1, 1], 0.1)


def test_choose_path_memory_cap():
    # sparse extras: qhat + khat, idx + rev_idx, rev_ptr, the selection workspace
    p = _p(heads=2)                    # NG = NB = 16, r = 16
    kph = [4, 4]
    ws = dsa.workspace_bytes(p, kph, dsa.DSA_WS_SELECT)
    extra = 2 * (16 + 16) * 16 * 4 + 2 * 16 * 8 * 4 + 2 * 17 * 4 + ws
    assert dsa.choose_path(p, kph, 0.1, extra) == dsa.PATH_SPARSE
    assert dsa.choose_path(p, kph, 0.1, extra - 1) == dsa.PATH_DENSE
    assert dsa.choose_path(p, kph, 0.1, 0) == dsa.PATH_SPARSE         # 0: no cap
    # kept lists beyond the sparse calls' index range: dense
    big = _p(heads=128, seq_len=64 * 8192, group=64)
    assert dsa.choose_path(big, [4096] * 128, 0.1) == dsa.PATH_DENSE
    assert dsa.choose_path(big, [8] * 128, 0.1) == dsa.PATH_SPARSE


def test_predictor_loss_grad_validation():
    lib = dsa.library()
    big = 1 << 40
    p = _p()
    pc = ctypes.byref(p.c())
    args = [FAKE] * 7     # Q, K, Wq, Wk, loss, dWq, dWk
    for i in range(7):
        bad = list(args)
        bad[i] = None
        assert lib.dsa_predictor_loss_grad(pc, *bad, FAKE, big, None) == -1, i
        bad[i] = ctypes.c_void_p(0x100004)
        assert lib.dsa_predictor_loss_grad(pc, *bad, FAKE, big, None) == -4, i
    need = dsa.workspace_bytes(p, None, dsa.DSA_WS_PRED_GRAD)
    # qbar, kbar, qhat, khat, E, Y, Z, row losses (16 groups x 16 blocks x 2 heads), each 256-byte aligned
    sections = [16 * 64, 16 * 64, 16 * 16, 16 * 16, 16 * 16, 16 * 16, 16 * 16, 16]
    partials = 4 * 2 * 2 * 16 * 64 * 16            # [H, W_q or W_k, 16 row ranges, d, r] fp32
    assert need == sum((4 * 2 * n + 255) // 256 * 256 for n in sections) + partials
    assert need == dsa.workspace_bytes(p, [1, 1], dsa.DSA_WS_PRED_GRAD)
    assert lib.dsa_predictor_loss_grad(pc, *args, FAKE, need - 1, None) == -6
    assert lib.dsa_predictor_loss_grad(pc, *args, None, big, None) == -6
    assert lib.dsa_predictor_loss_grad(pc, *args, ctypes.c_void_p(0x100008), big, None) == -4
    assert lib.dsa_predictor_loss_grad(ctypes.byref(_p(rank=12).c()), *args, FAKE, big, None) == -5
    assert lib.dsa_predictor_loss_grad(None, *args, FAKE, big, None) == -1


def test_coverage_calls_validation():
    lib = dsa.library()
    big = 1 << 40
    p = _p()
    pc = ctypes.byref(p.c())
    kph = dsa._kph([4, 4])
    # select: scores, qhat, khat, kph, coverage, idx, cnt, rev_ptr, rev_idx, dump, ws, bytes, stream
    sel = lambda cov, cnt, ws=FAKE: lib.dsa_select_coverage_blocks(pc, FAKE, FAKE, FAKE, kph, cov, FAKE, cnt, FAKE,
                                                                   FAKE, None, ws, big, None)
    for cov in (0.0, -0.5, 1.0000001, float("nan")):
        assert sel(cov, FAKE) == -1, cov
    assert sel(0.9, None) == -1
    assert sel(0.9, ctypes.c_void_p(0x100004)) == -4
    assert sel(0.9, FAKE, None) == -6
    assert lib.dsa_select_coverage_blocks(pc, FAKE, FAKE, FAKE, dsa._kph([0, 4]), 0.9, FAKE, FAKE, FAKE, FAKE, None,
                                          FAKE, big, None) == -2
    # forward / backward with counts
    assert lib.dsa_sparse_attn_fwd_varlen(pc, FAKE, FAKE, FAKE, FAKE, None, kph, FAKE, FAKE, FAKE, big, None) == -1
    assert lib.dsa_sparse_attn_fwd_varlen(pc, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x100004), kph, FAKE, FAKE,
                                          FAKE, big, None) == -4
    assert lib.dsa_sparse_attn_fwd_varlen(pc, FAKE, FAKE, FAKE, None, FAKE, kph, FAKE, FAKE, FAKE, big, None) == -1
    args = [FAKE] * 6 + [FAKE, None, kph] + [FAKE] * 5
    assert lib.dsa_sparse_attn_bwd_varlen(pc, *args, FAKE, big, None) == -1
    args[7] = ctypes.c_void_p(0x100004)
    assert lib.dsa_sparse_attn_bwd_varlen(pc, *args, FAKE, big, None) == -4
    args[7] = FAKE
    f32 = ctypes.byref(_p(dtype=dsa.DSA_F32).c())
    assert lib.dsa_sparse_attn_bwd_varlen(f32, *args, FAKE, big, None) == -3


def test_select_blocks_validation():
    lib = dsa.library()
    big = 1 << 40

    def call(p, kph, cov, flags, cnt=FAKE):
        return lib.dsa_select_blocks(ctypes.byref(p.c()), FAKE, FAKE, FAKE, dsa._kph(kph), cov, flags, FAKE, cnt, FAKE,
                                     FAKE, None, FAKE, big, None)
    p64, p128 = _p(), _p(group=128)
    assert call(p64, [4, 4], 0.0, 2) == -1                  # unknown flag
    assert call(p64, [4, 4], -0.1, 0) == -1
    assert call(p64, [4, 4], 1.5, 0) == -1
    assert call(p64, [4, 4], float("nan"), 0) == -1
    assert call(p64, [4, 4], 0.5, 0, None) == -1            # coverage needs the counts
    assert call(p64, [4, 4], 0.5, 0, ctypes.c_void_p(0x100004)) == -4
    assert call(p128, [1, 4], 0.0, dsa.SELECT_DIAGONAL) == -2   # G = 128 forces two blocks: k_h >= 2
    assert lib.dsa_select_blocks(ctypes.byref(p64.c()), FAKE, FAKE, FAKE, dsa._kph([4, 4]), 0.0, 0, FAKE, None, FAKE,
                                 FAKE, None, None, 0, None) == -6


def test_pooled_scores_validation():
    lib = dsa.library()
    big = 1 << 40
    p = _p()
    pc = ctypes.byref(p.c())
    call = lambda pooling, *a: lib.dsa_predict_block_scores_pooled(pc, *a[:4], pooling, a[4], a[5], big, None)
    args = [FAKE] * 6
    for bad_pool in (0, 3, -1):
        assert call(bad_pool, *args) == -1
    for i in range(5):
        bad = list(args)
        bad[i] = None
        assert call(dsa.POOL_MAX, *bad) == -1, i
        bad[i] = ctypes.c_void_p(0x100004)
        assert call(dsa.POOL_LSE, *bad) == -4, i
    need = dsa.workspace_bytes(p, None, dsa.DSA_WS_PRED_POOLED)
    assert need == 2 * ((2 * 1024 * 16 * 2 + 255) // 256 * 256)       # fp16 projections of Q and K
    assert lib.dsa_predict_block_scores_pooled(pc, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, need - 1, None) == -6
    assert lib.dsa_predict_block_scores_pooled(pc, FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, big, None) == -6


def test_noalloc_select_rejects_problems_beyond_its_scratch():
    # 520,000 tokens, 24 heads, 840 kept blocks per row: the selection's scratch would be ~655 MB
    lib = dsa.library()
    p = dsa.Problem(batch=1, heads=24, seq_len=8125 * 64, head_dim=128, rank=32, group=64)
    kph = dsa._kph([840] * 24)
    st = lib.dsa_select_topk_blocks_noalloc(ctypes.byref(p.c()), FAKE, None, None, kph, FAKE, FAKE, FAKE, None, None)
    assert st == -8 and "scratch" in dsa.status_string(st)
    # and the usual validation comes first
    assert lib.dsa_select_topk_blocks_noalloc(ctypes.byref(p.c()), None, None, None, kph, FAKE, FAKE, FAKE, None,
                                              None) == -1
