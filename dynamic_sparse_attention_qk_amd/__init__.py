"""MI355X (gfx950) dynamic sparse attention: Python binding of libdsa.so.

The four calls of the C ABI (include/dsa.h) are exposed under the same names
and take torch tensors only as holders of device memory: each wrapper checks
that the tensors are laid out as the ABI expects, passes their pointers and the
current HIP stream, and raises on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.

    predict_block_scores  low-rank predictor -> qhat, khat (and scores)
    select_topk_blocks    top-k kept blocks per (head, group) + reverse index
    sparse_attn_fwd       attention over the kept blocks -> O, LSE
    sparse_attn_bwd       dQ, dK, dV for the fixed selection

``SparseAttentionPlan`` allocates the outputs and workspaces of one problem
with torch and runs the calls in order.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_F32, DSA_BF16 = 0, 1
DSA_WS_SELECT, DSA_WS_BWD, DSA_WS_FWD, DSA_WS_PRED_GRAD, DSA_WS_PRED_POOLED = 0, 1, 2, 3, 4


class DsaError(RuntimeError):
    def __init__(self, call: str, status: int, text: str):
        super().__init__(f"{call} failed: status {status} ({text})")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "seq_len", "head_dim", "rank", "group", "block", "dtype")]


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libdsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m dynamic_sparse_attention_qk_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32p, i64p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p
        pp = ctypes.POINTER(_Problem)
        kph = ctypes.POINTER(ctypes.c_int32)
        lib.dsa_version.restype = ctypes.c_char_p
        lib.dsa_status_string.restype = ctypes.c_char_p
        lib.dsa_status_string.argtypes = [ctypes.c_int]
        lib.dsa_index_layout.argtypes = [pp, kph, i64p]
        lib.dsa_workspace_bytes.restype = ctypes.c_size_t
        lib.dsa_workspace_bytes.argtypes = [pp, kph, ctypes.c_int]
        lib.dsa_predict_block_scores.argtypes = [pp, vp, vp, f32p, f32p, f32p, f32p, f32p, vp]
        lib.dsa_select_topk_blocks.argtypes = [pp, f32p, f32p, f32p, kph, i32p, i32p, i32p, f32p, vp,
                                               ctypes.c_size_t, vp]
        lib.dsa_sparse_attn_fwd.argtypes = [pp, vp, vp, vp, i32p, kph, f32p, f32p, vp, ctypes.c_size_t, vp]
        lib.dsa_sparse_attn_bwd.argtypes = [pp, vp, vp, vp, f32p, vp, f32p, i32p, kph, i32p, i32p, f32p, f32p,
                                            f32p, vp, ctypes.c_size_t, vp]
        sz = ctypes.c_size_t
        lib.dsa_sparse_attn_bwd_preprocess.argtypes = [pp, vp, vp, vp, f32p, vp, f32p, vp, sz, vp]
        lib.dsa_sparse_attn_bwd_dkdv.argtypes = [pp, kph, i32p, i32p, f32p, f32p, vp, sz, vp]
        lib.dsa_sparse_attn_bwd_dq.argtypes = [pp, i32p, kph, f32p, vp, sz, vp]
        lib.dsa_sparse_attn_fwd_split.argtypes = [pp, vp, vp, vp, i32p, kph, ctypes.c_int, f32p, f32p, vp, sz, vp]
        lib.dsa_attn_merge.argtypes = [pp, ctypes.c_int, f32p, f32p, f32p, f32p, vp]
        lib.dsa_dense_attn_fwd.argtypes = [pp, vp, vp, vp, f32p, f32p, vp, sz, vp]
        lib.dsa_dense_attn_bwd.argtypes = [pp, vp, vp, vp, f32p, vp, f32p, f32p, f32p, f32p, vp, sz, vp]
        lib.dsa_choose_path.argtypes = [pp, kph, ctypes.c_double, sz]
        lib.dsa_predictor_loss_grad.argtypes = [pp, vp, vp, f32p, f32p, f32p, f32p, f32p, vp, sz, vp]
        lib.dsa_select_coverage_blocks.argtypes = [pp, f32p, f32p, f32p, kph, ctypes.c_double, i32p, i32p, i32p,
                                                   i32p, f32p, vp, sz, vp]
        lib.dsa_sparse_attn_fwd_varlen.argtypes = [pp, vp, vp, vp, i32p, i32p, kph, f32p, f32p, vp, sz, vp]
        lib.dsa_predict_block_scores_pooled.argtypes = [pp, vp, vp, f32p, f32p, ctypes.c_int, f32p, vp, sz, vp]
        lib.dsa_select_blocks.argtypes = [pp, f32p, f32p, f32p, kph, ctypes.c_double, ctypes.c_int, i32p, i32p, i32p,
                                          i32p, f32p, vp, sz, vp]
        lib.dsa_sparse_attn_bwd_varlen.argtypes = [pp, vp, vp, vp, f32p, vp, f32p, i32p, i32p, kph, i32p, i32p,
                                                   f32p, f32p, f32p, vp, sz, vp]
        for name in ("dsa_index_layout", "dsa_predict_block_scores", "dsa_select_topk_blocks",
                     "dsa_sparse_attn_fwd", "dsa_sparse_attn_bwd", "dsa_sparse_attn_bwd_preprocess",
                     "dsa_sparse_attn_bwd_dkdv", "dsa_sparse_attn_bwd_dq", "dsa_sparse_attn_fwd_split",
                     "dsa_attn_merge", "dsa_dense_attn_fwd", "dsa_dense_attn_bwd", "dsa_choose_path",
                     "dsa_predictor_loss_grad", "dsa_select_coverage_blocks", "dsa_sparse_attn_fwd_varlen",
                     "dsa_sparse_attn_bwd_varlen", "dsa_select_blocks", "dsa_predict_block_scores_pooled"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


EXPORTED = ("dsa_version", "dsa_status_string", "dsa_index_layout", "dsa_workspace_bytes",
            "dsa_predict_block_scores", "dsa_select_topk_blocks", "dsa_sparse_attn_fwd", "dsa_sparse_attn_bwd",
            "dsa_sparse_attn_bwd_preprocess", "dsa_sparse_attn_bwd_dkdv", "dsa_sparse_attn_bwd_dq",
            "dsa_sparse_attn_fwd_split", "dsa_attn_merge", "dsa_dense_attn_fwd", "dsa_dense_attn_bwd",
            "dsa_choose_path", "dsa_predictor_loss_grad", "dsa_select_coverage_blocks", "dsa_sparse_attn_fwd_varlen",
            "dsa_sparse_attn_bwd_varlen", "dsa_select_blocks", "dsa_predict_block_scores_pooled")
SELECT_DIAGONAL = 1  # DSA_SELECT_DIAGONAL
POOL_MAX, POOL_LSE = 1, 2  # DSA_POOL_MAX, DSA_POOL_LSE
MAX_SPLIT = 64  # DSA_MAX_SPLIT
PATH_DENSE, PATH_SPARSE = 0, 1  # dsa_path
DEFAULT_MIN_SPARSITY = 0.06     # DSA_DEFAULT_MIN_SPARSITY


@dataclass(frozen=True)
class Problem:
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    rank: int
    group: int
    block: int = 64
    dtype: int = DSA_BF16

    def c(self) -> _Problem:
        return _Problem(self.batch, self.heads, self.seq_len, self.head_dim, self.rank, self.group, self.block,
                        self.dtype)

    @property
    def n_groups(self) -> int:
        return self.seq_len // self.group

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block


def _kph(k_per_head: Sequence[int]):
    arr = (ctypes.c_int32 * len(k_per_head))(*[int(x) for x in k_per_head])
    return arr


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdsa must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(call: str, status: int):
    if status != 0:
        raise DsaError(call, status, library().dsa_status_string(status).decode())


def status_string(status: int) -> str:
    return library().dsa_status_string(status).decode()


def version() -> str:
    return library().dsa_version().decode()


def index_layout(p: Problem, k_per_head: Sequence[int]) -> np.ndarray:
    """Host int64 [B*H + 1] offsets of each (b, h) region of the kept-block list."""
    out = np.zeros(p.batch * p.heads + 1, dtype=np.int64)
    _check("dsa_index_layout", library().dsa_index_layout(
        ctypes.byref(p.c()), _kph(k_per_head), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
    return out


def workspace_bytes(p: Problem, k_per_head: Optional[Sequence[int]], which: int) -> int:
    """Workspace bytes of a call; k_per_head may be None for DSA_WS_FWD / DSA_WS_BWD / DSA_WS_PRED_GRAD."""
    kph = None if k_per_head is None else _kph(k_per_head)
    return int(library().dsa_workspace_bytes(ctypes.byref(p.c()), kph, which))


def predict_block_scores(p: Problem, Q, K, Wq, Wk, qhat, khat, scores=None, stream=None) -> None:
    _check("dsa_predict_block_scores", library().dsa_predict_block_scores(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), _ptr(qhat), _ptr(khat), _ptr(scores),
        _stream(stream)))


def select_topk_blocks(p: Problem, scores, qhat, khat, k_per_head, idx, rev_ptr, rev_idx, workspace,
                       scores_dump=None, stream=None) -> None:
    _check("dsa_select_topk_blocks", library().dsa_select_topk_blocks(
        ctypes.byref(p.c()), _ptr(scores), _ptr(qhat), _ptr(khat), _kph(k_per_head), _ptr(idx), _ptr(rev_ptr),
        _ptr(rev_idx), _ptr(scores_dump), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def select_coverage_blocks(p: Problem, scores, qhat, khat, k_per_head, coverage: float, idx, cnt, rev_ptr, rev_idx,
                           workspace, scores_dump=None, stream=None) -> None:
    """Per row, the shortest run of blocks in score order whose estimated attention mass reaches coverage
    (at most k_h); counts to cnt [B, H, NG]."""
    _check("dsa_select_coverage_blocks", library().dsa_select_coverage_blocks(
        ctypes.byref(p.c()), _ptr(scores), _ptr(qhat), _ptr(khat), _kph(k_per_head), float(coverage), _ptr(idx),
        _ptr(cnt), _ptr(rev_ptr), _ptr(rev_idx), _ptr(scores_dump), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def predict_block_scores_pooled(p: Problem, Q, K, Wq, Wk, pooling: int, scores, workspace, stream=None) -> None:
    """Block scores pooled from the token-level low-rank logits (POOL_MAX or POOL_LSE)."""
    _check("dsa_predict_block_scores_pooled", library().dsa_predict_block_scores_pooled(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), int(pooling), _ptr(scores), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def select_blocks(p: Problem, scores, qhat, khat, k_per_head, coverage: float, flags: int, idx, cnt, rev_ptr,
                  rev_idx, workspace, scores_dump=None, stream=None) -> None:
    """The general selection: top-k (coverage 0) or by coverage, optionally with the diagonal forced."""
    _check("dsa_select_blocks", library().dsa_select_blocks(
        ctypes.byref(p.c()), _ptr(scores), _ptr(qhat), _ptr(khat), _kph(k_per_head), float(coverage), int(flags),
        _ptr(idx), _ptr(cnt), _ptr(rev_ptr), _ptr(rev_idx), _ptr(scores_dump), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def sparse_attn_fwd_varlen(p: Problem, Q, K, V, idx, cnt, k_per_head, O, LSE, workspace=None, stream=None) -> None:
    nbytes = 0 if workspace is None else _nbytes(workspace)
    _check("dsa_sparse_attn_fwd_varlen", library().dsa_sparse_attn_fwd_varlen(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(cnt), _kph(k_per_head), _ptr(O), _ptr(LSE),
        _ptr(workspace), nbytes, _stream(stream)))


def sparse_attn_bwd_varlen(p: Problem, Q, K, V, O, dO, LSE, idx, cnt, k_per_head, rev_ptr, rev_idx, dQ, dK, dV,
                           workspace, stream=None) -> None:
    _check("dsa_sparse_attn_bwd_varlen", library().dsa_sparse_attn_bwd_varlen(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(idx), _ptr(cnt),
        _kph(k_per_head), _ptr(rev_ptr), _ptr(rev_idx), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def sparse_attn_fwd(p: Problem, Q, K, V, idx, k_per_head, O, LSE, workspace=None, stream=None) -> None:
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_attn_fwd", library().dsa_sparse_attn_fwd(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _kph(k_per_head), _ptr(O), _ptr(LSE),
        _ptr(workspace), nbytes, _stream(stream)))


def sparse_attn_fwd_split(p: Problem, Q, K, V, idx, k_per_head, n_split: int, O_part, LSE_part, workspace=None,
                          stream=None) -> None:
    """Partial states over n_split contiguous parts of every row's kept list: O_part [n_split, B, H, N, d],
    LSE_part [n_split, B, H, N] (fp32)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_attn_fwd_split", library().dsa_sparse_attn_fwd_split(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _kph(k_per_head), int(n_split), _ptr(O_part),
        _ptr(LSE_part), _ptr(workspace), nbytes, _stream(stream)))


def attn_merge(p: Problem, n_parts: int, O_part, LSE_part, O, LSE, stream=None) -> None:
    """O, LSE from n_parts partial states (log-sum-exp weighted)."""
    _check("dsa_attn_merge", library().dsa_attn_merge(
        ctypes.byref(p.c()), int(n_parts), _ptr(O_part), _ptr(LSE_part), _ptr(O), _ptr(LSE), _stream(stream)))


def dense_attn_fwd(p: Problem, Q, K, V, O, LSE, workspace=None, stream=None) -> None:
    """Full attention over every key (the dispatcher's dense branch)."""
    nbytes = 0 if workspace is None else _nbytes(workspace)
    _check("dsa_dense_attn_fwd", library().dsa_dense_attn_fwd(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), _ptr(workspace), nbytes,
        _stream(stream)))


def dense_attn_bwd(p: Problem, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, stream=None) -> None:
    _check("dsa_dense_attn_bwd", library().dsa_dense_attn_bwd(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def predictor_loss_grad(p: Problem, Q, K, Wq, Wk, loss, dWq, dWk, workspace, stream=None) -> None:
    """Stage-1 predictor training: loss [H] and its gradients dWq, dWk [H, d, r] (all fp32)."""
    _check("dsa_predictor_loss_grad", library().dsa_predictor_loss_grad(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(Wq), _ptr(Wk), _ptr(loss), _ptr(dWq), _ptr(dWk), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def choose_path(p: Problem, k_per_head: Sequence[int], min_sparsity: float = -1.0, max_sparse_bytes: int = 0) -> int:
    """PATH_SPARSE or PATH_DENSE for one layer (min_sparsity < 0: the library's measured default)."""
    st = library().dsa_choose_path(ctypes.byref(p.c()), _kph(k_per_head), float(min_sparsity), int(max_sparse_bytes))
    if st < 0:
        _check("dsa_choose_path", st)
    return st


def sparse_attn_bwd(p: Problem, Q, K, V, O, dO, LSE, idx, k_per_head, rev_ptr, rev_idx, dQ, dK, dV, workspace,
                    stream=None) -> None:
    _check("dsa_sparse_attn_bwd", library().dsa_sparse_attn_bwd(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(idx), _kph(k_per_head),
        _ptr(rev_ptr), _ptr(rev_idx), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def sparse_attn_bwd_preprocess(p: Problem, Q, K, V, O, dO, LSE, workspace, stream=None) -> None:
    _check("dsa_sparse_attn_bwd_preprocess", library().dsa_sparse_attn_bwd_preprocess(
        ctypes.byref(p.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def sparse_attn_bwd_dkdv(p: Problem, k_per_head, rev_ptr, rev_idx, dK, dV, workspace, stream=None) -> None:
    _check("dsa_sparse_attn_bwd_dkdv", library().dsa_sparse_attn_bwd_dkdv(
        ctypes.byref(p.c()), _kph(k_per_head), _ptr(rev_ptr), _ptr(rev_idx), _ptr(dK), _ptr(dV), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def sparse_attn_bwd_dq(p: Problem, idx, k_per_head, dQ, workspace, stream=None) -> None:
    _check("dsa_sparse_attn_bwd_dq", library().dsa_sparse_attn_bwd_dq(
        ctypes.byref(p.c()), _ptr(idx), _kph(k_per_head), _ptr(dQ), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


class SparseAttentionPlan:
    """Outputs and workspaces of one problem, allocated once with torch, plus the calls in order."""

    def __init__(self, p: Problem, k_per_head: Sequence[int], device="cuda", materialise_scores: bool = True,
                 backward: bool = True, coverage: Optional[float] = None, select_flags: int = 0):
        """coverage: select by attention coverage (k_per_head is then each row's capacity) and run the
        per-row-count forward and backward; select_flags: SELECT_DIAGONAL keeps each group's own blocks."""
        self.p = p
        self.k_per_head = [int(x) for x in k_per_head]
        self.coverage = coverage
        self.select_flags = int(select_flags)
        self.cnt = (torch.empty(p.batch, p.heads, p.n_groups, dtype=torch.int32, device=device)
                    if coverage is not None else None)
        self.row_base = index_layout(p, self.k_per_head)
        total = int(self.row_base[-1])
        B, H, N, D, R = p.batch, p.heads, p.seq_len, p.head_dim, p.rank
        f32 = dict(dtype=torch.float32, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.qhat = torch.empty(B, H, p.n_groups, R, **f32)
        self.khat = torch.empty(B, H, p.n_blocks, R, **f32)
        self.scores = torch.empty(B, H, p.n_groups, p.n_blocks, **f32) if materialise_scores else None
        self.idx = torch.empty(max(total, 1), **i32)
        self.rev_ptr = torch.empty(B * H, p.n_blocks + 1, **i32)
        self.rev_idx = torch.empty(max(total, 1), **i32)
        self.ws_select = torch.empty(workspace_bytes(p, self.k_per_head, DSA_WS_SELECT), dtype=torch.uint8,
                                     device=device)
        self.ws_fwd = torch.empty(max(workspace_bytes(p, self.k_per_head, DSA_WS_FWD), 16), dtype=torch.uint8,
                                  device=device)
        self.O = torch.empty(B, H, N, D, **f32)
        self.LSE = torch.empty(B, H, N, **f32)
        if backward:
            self.dQ = torch.empty(B, H, N, D, **f32)
            self.dK = torch.empty(B, H, N, D, **f32)
            self.dV = torch.empty(B, H, N, D, **f32)
            self.ws_bwd = torch.empty(workspace_bytes(p, self.k_per_head, DSA_WS_BWD), dtype=torch.uint8,
                                      device=device)

    def predict(self, Q, K, Wq, Wk, stream=None):
        predict_block_scores(self.p, Q, K, Wq, Wk, self.qhat, self.khat, self.scores, stream)

    def select(self, stream=None, scores_dump=None):
        if self.select_flags:
            select_blocks(self.p, self.scores, self.qhat, self.khat, self.k_per_head,
                          0.0 if self.coverage is None else self.coverage, self.select_flags, self.idx, self.cnt,
                          self.rev_ptr, self.rev_idx, self.ws_select, scores_dump=scores_dump, stream=stream)
        elif self.coverage is not None:
            select_coverage_blocks(self.p, self.scores, self.qhat, self.khat, self.k_per_head, self.coverage,
                                   self.idx, self.cnt, self.rev_ptr, self.rev_idx, self.ws_select,
                                   scores_dump=scores_dump, stream=stream)
        else:
            select_topk_blocks(self.p, self.scores, self.qhat, self.khat, self.k_per_head, self.idx, self.rev_ptr,
                               self.rev_idx, self.ws_select, scores_dump=scores_dump, stream=stream)

    def forward(self, Q, K, V, stream=None):
        if self.cnt is not None:
            sparse_attn_fwd_varlen(self.p, Q, K, V, self.idx, self.cnt, self.k_per_head, self.O, self.LSE,
                                   self.ws_fwd, stream)
        else:
            sparse_attn_fwd(self.p, Q, K, V, self.idx, self.k_per_head, self.O, self.LSE, self.ws_fwd, stream)

    def backward(self, Q, K, V, dO, stream=None):
        if self.cnt is not None:
            sparse_attn_bwd_varlen(self.p, Q, K, V, self.O, dO, self.LSE, self.idx, self.cnt, self.k_per_head,
                                   self.rev_ptr, self.rev_idx, self.dQ, self.dK, self.dV, self.ws_bwd, stream)
        else:
            sparse_attn_bwd(self.p, Q, K, V, self.O, dO, self.LSE, self.idx, self.k_per_head, self.rev_ptr,
                            self.rev_idx, self.dQ, self.dK, self.dV, self.ws_bwd, stream)

    def backward_stages(self, Q, K, V, dO, stream=None):
        """The backward as its three stages (same result as backward()); top-k selection only."""
        if self.cnt is not None:
            raise ValueError("the staged backward takes no per-row counts: use backward()")
        sparse_attn_bwd_preprocess(self.p, Q, K, V, self.O, dO, self.LSE, self.ws_bwd, stream)
        sparse_attn_bwd_dkdv(self.p, self.k_per_head, self.rev_ptr, self.rev_idx, self.dK, self.dV, self.ws_bwd,
                             stream)
        sparse_attn_bwd_dq(self.p, self.idx, self.k_per_head, self.dQ, self.ws_bwd, stream)

    def step(self, Q, K, V, Wq, Wk, dO=None, stream=None):
        """predict -> select -> fwd (-> bwd): one pass of the whole hot path."""
        self.predict(Q, K, Wq, Wk, stream)
        self.select(stream)
        self.forward(Q, K, V, stream)
        if dO is not None:
            self.backward(Q, K, V, dO, stream)

    def idx_rows(self, b: int, h: int) -> torch.Tensor:
        """View of the kept-block list of (b, h) as [NG, k_h]."""
        s = int(self.row_base[b * self.p.heads + h])
        return self.idx[s:s + self.p.n_groups * self.k_per_head[h]].view(self.p.n_groups, self.k_per_head[h])


class DenseAttentionPlan:
    """Outputs and workspaces of full attention for one problem (the dispatcher's dense branch)."""

    def __init__(self, p: Problem, device="cuda", backward: bool = True):
        self.p = p
        B, H, N, D = p.batch, p.heads, p.seq_len, p.head_dim
        f32 = dict(dtype=torch.float32, device=device)
        self.ws_fwd = torch.empty(max(workspace_bytes(p, None, DSA_WS_FWD), 16), dtype=torch.uint8, device=device)
        self.O = torch.empty(B, H, N, D, **f32)
        self.LSE = torch.empty(B, H, N, **f32)
        if backward:
            self.dQ = torch.empty(B, H, N, D, **f32)
            self.dK = torch.empty(B, H, N, D, **f32)
            self.dV = torch.empty(B, H, N, D, **f32)
            self.ws_bwd = torch.empty(workspace_bytes(p, None, DSA_WS_BWD), dtype=torch.uint8, device=device)

    def forward(self, Q, K, V, stream=None):
        dense_attn_fwd(self.p, Q, K, V, self.O, self.LSE, self.ws_fwd, stream)

    def backward(self, Q, K, V, dO, stream=None):
        dense_attn_bwd(self.p, Q, K, V, self.O, dO, self.LSE, self.dQ, self.dK, self.dV, self.ws_bwd, stream)
