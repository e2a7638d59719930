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
# DSA_LIBRARY selects another build of the same library (libdsa_debug.so: list checks; libdsa_san.so: host code
# under AddressSanitizer and UndefinedBehaviorSanitizer), by name within the package or as a path
LIB_PATH = os.path.join(_PKG, os.environ.get("DSA_LIBRARY", "libdsa.so"))

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
    """The loaded libdsa.so (or the build DSA_LIBRARY names); raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Loads one build of the library (path, or a name within the package) with the C signatures set."""
    if not os.path.isabs(path):
        path = os.path.join(_PKG, path)
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m dynamic_sparse_attention_qk_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
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
    lib.dsa_select_topk_blocks_noalloc.argtypes = [pp, f32p, f32p, f32p, kph, i32p, i32p, i32p, f32p, vp]
    lib.dsa_sparse_attn_fwd.argtypes = [pp, vp, vp, vp, i32p, kph, f32p, f32p, vp, ctypes.c_size_t, vp]
    lib.dsa_sparse_attn_bwd.argtypes = [pp, vp, vp, vp, f32p, vp, f32p, i32p, kph, i32p, i32p, f32p, f32p,
                                        f32p, vp, ctypes.c_size_t, vp]
    sz = ctypes.c_size_t
    lib.dsa_sparse_attn_bwd_ex.argtypes = [pp, vp, vp, vp, f32p, vp, f32p, i32p, kph, i32p, i32p, f32p, f32p,
                                           f32p, ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.dsa_sparse_attn_bwd_preprocess.argtypes = [pp, vp, vp, vp, f32p, vp, f32p, vp, sz, vp]
    lib.dsa_sparse_attn_bwd_preprocess_ex.argtypes = [pp, vp, vp, vp, f32p, vp, f32p, ctypes.c_int, vp, sz, vp]
    lib.dsa_sparse_attn_bwd_dkdv.argtypes = [pp, vp, vp, vp, vp, kph, i32p, i32p, f32p, f32p, vp, sz, vp]
    lib.dsa_sparse_attn_bwd_dq.argtypes = [pp, vp, vp, i32p, kph, f32p, vp, sz, vp]
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
                 "dsa_sparse_attn_bwd_varlen", "dsa_select_blocks", "dsa_predict_block_scores_pooled",
                 "dsa_select_topk_blocks_noalloc", "dsa_sparse_attn_bwd_ex",
                 "dsa_sparse_attn_bwd_preprocess_ex"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


EXPORTED = ("dsa_version", "dsa_status_string", "dsa_index_layout", "dsa_workspace_bytes",
            "dsa_predict_block_scores", "dsa_select_topk_blocks", "dsa_sparse_attn_fwd", "dsa_sparse_attn_bwd",
            "dsa_sparse_attn_bwd_preprocess", "dsa_sparse_attn_bwd_dkdv", "dsa_sparse_attn_bwd_dq",
            "dsa_sparse_attn_fwd_split", "dsa_attn_merge", "dsa_dense_attn_fwd", "dsa_dense_attn_bwd",
            "dsa_choose_path", "dsa_predictor_loss_grad", "dsa_select_coverage_blocks", "dsa_sparse_attn_fwd_varlen",
            "dsa_sparse_attn_bwd_varlen", "dsa_select_blocks", "dsa_predict_block_scores_pooled",
            "dsa_select_topk_blocks_noalloc", "dsa_sparse_attn_bwd_ex", "dsa_sparse_attn_bwd_preprocess_ex")
BWD_V_FROM_FORWARD = 1  # DSA_BWD_V_FROM_FORWARD
NOALLOC_SCRATCH_BYTES = 16 << 20  # DSA_NOALLOC_SCRATCH_BYTES
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

    @property
    def rows(self) -> int:
        """B * H * N: rows of O, LSE and every [B, H, N, d] tensor."""
        return self.batch * self.heads * self.seq_len

    @property
    def elems(self) -> int:
        """B * H * N * d: elements of Q, K, V, dO, O, dQ, dK, dV."""
        return self.rows * self.head_dim

    def list_len(self, k_per_head: Sequence[int]) -> int:
        """Entries of the kept-block list (and of the reverse list): B * NG * sum_h k_h."""
        return self.batch * self.n_groups * int(sum(int(x) for x in k_per_head))




def _kph(k_per_head: Sequence[int], heads: Optional[int] = None):
    """Host int32 array of the kept counts; with ``heads``, its length must equal the head count."""
    if heads is not None and len(k_per_head) != heads:
        raise ValueError(f"k_per_head has {len(k_per_head)} entries for {heads} heads")
    return (ctypes.c_int32 * len(k_per_head))(*[int(x) for x in k_per_head])


_I32, _F32 = torch.int32, torch.float32


def _io(p: "Problem"):
    """torch dtype of Q, K, V, dO for the problem."""
    return torch.bfloat16 if p.dtype == DSA_BF16 else torch.float32


class _Args:
    """Pointers for one library call, after checking what the C ABI cannot: dtype, size, layout, device.

    The ABI receives bare pointers, so a short tensor or one of the wrong dtype would let the kernels read or
    write past an allocation; every such mismatch raises here instead.  dtype, size and layout are checked as
    each argument is added, the device of all of them when the call is made (so every other mismatch is
    reported first, also for host tensors).
    """

    def __init__(self, p: "Problem"):
        self.p = p
        self._tensors = []

    def t(self, t: Optional[torch.Tensor], name: str, dtype=None, numel: Optional[int] = None,
          required: bool = True):
        if t is None:
            if required:
                raise ValueError(f"{name} is required")
            return None
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if numel is not None and t.numel() < numel:
            raise ValueError(f"{name} holds {t.numel()} elements, the problem needs {numel}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors passed to libdsa must be contiguous")
        self._tensors.append((name, t))
        return ctypes.c_void_p(t.data_ptr())

    # tensors whose sizes the problem fixes
    def io(self, t, name, required=True):          # Q, K, V, dO: [B, H, N, d] in the problem's dtype
        return self.t(t, name, _io(self.p), self.p.elems, required)

    def f32(self, t, name, numel, required=True):
        return self.t(t, name, _F32, numel, required)

    def out(self, t, name, parts=1):              # O, dQ, dK, dV (per part): [B, H, N, d] fp32
        return self.t(t, name, _F32, parts * self.p.elems)

    def rows(self, t, name, parts=1):             # LSE (per part): [B, H, N] fp32
        return self.t(t, name, _F32, parts * self.p.rows)

    def weights(self, t, name):                   # Wq, Wk, dWq, dWk: [H, d, r] fp32
        p = self.p
        return self.t(t, name, _F32, p.heads * p.head_dim * p.rank)

    def scores(self, t, name="scores", required=False):
        p = self.p
        return self.t(t, name, _F32, p.batch * p.heads * p.n_groups * p.n_blocks, required)

    def qhat(self, t, required=False):
        p = self.p
        return self.t(t, "qhat", _F32, p.batch * p.heads * p.n_groups * p.rank, required)

    def khat(self, t, required=False):
        p = self.p
        return self.t(t, "khat", _F32, p.batch * p.heads * p.n_blocks * p.rank, required)

    def idx(self, t, kph, name="idx"):            # kept-block list / reverse list: B * NG * sum k_h int32
        return self.t(t, name, _I32, self.p.list_len(kph))

    def rev_ptr(self, t):
        p = self.p
        return self.t(t, "rev_ptr", _I32, p.batch * p.heads * (p.n_blocks + 1))

    def cnt(self, t, required=True):
        p = self.p
        return self.t(t, "cnt", _I32, p.batch * p.heads * p.n_groups, required)

    def ws(self, t, required=True):
        """A workspace: any dtype; its byte count goes to the library, which checks it against the call."""
        return self.t(t, "workspace", None, None, required), _nbytes(t)

    def call(self, fn: str, *args, stream=None) -> int:
        """Checks that every tensor is on the GPU, then calls libdsa's ``fn`` with ``args`` and the stream (the
        current one if None) last; raises on a negative status."""
        for name, t in self._tensors:
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
        st = getattr(library(), fn)(*args, _stream(stream))
        if st < 0:
            _check(fn, st)
        return st


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


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
        ctypes.byref(p.c()), _kph(k_per_head, p.heads), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
    return out


def workspace_bytes(p: Problem, k_per_head: Optional[Sequence[int]], which: int) -> int:
    """Workspace bytes of a call; k_per_head may be None for DSA_WS_FWD / DSA_WS_BWD / DSA_WS_PRED_GRAD."""
    kph = None if k_per_head is None else _kph(k_per_head, p.heads)
    return int(library().dsa_workspace_bytes(ctypes.byref(p.c()), kph, which))


def predict_block_scores(p: Problem, Q, K, Wq, Wk, qhat, khat, scores=None, stream=None) -> None:
    a = _Args(p)
    a.call("dsa_predict_block_scores", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.weights(Wq, "Wq"),
           a.weights(Wk, "Wk"), a.qhat(qhat, True), a.khat(khat, True), a.scores(scores), stream=stream)


def predict_block_scores_pooled(p: Problem, Q, K, Wq, Wk, pooling: int, scores, workspace, stream=None) -> None:
    """Block scores pooled from the token-level low-rank logits (POOL_MAX or POOL_LSE)."""
    a = _Args(p)
    a.call("dsa_predict_block_scores_pooled", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"),
           a.weights(Wq, "Wq"), a.weights(Wk, "Wk"), int(pooling), a.scores(scores, required=True), *a.ws(workspace),
           stream=stream)


def select_topk_blocks(p: Problem, scores, qhat, khat, k_per_head, idx, rev_ptr, rev_idx, workspace,
                       scores_dump=None, stream=None) -> None:
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_select_topk_blocks", ctypes.byref(p.c()), a.scores(scores), a.qhat(qhat), a.khat(khat), kph,
           a.idx(idx, k_per_head), a.rev_ptr(rev_ptr), a.idx(rev_idx, k_per_head, "rev_idx"),
           a.scores(scores_dump, "scores_dump"), *a.ws(workspace), stream=stream)


def select_topk_blocks_noalloc(p: Problem, scores, qhat, khat, k_per_head, idx, rev_ptr, rev_idx, scores_dump=None,
                               stream=None) -> None:
    """select_topk_blocks without a workspace (the library's static per-GPU scratch; calls that overlap on one
    GPU race)."""
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_select_topk_blocks_noalloc", ctypes.byref(p.c()), a.scores(scores), a.qhat(qhat), a.khat(khat), kph,
           a.idx(idx, k_per_head), a.rev_ptr(rev_ptr), a.idx(rev_idx, k_per_head, "rev_idx"),
           a.scores(scores_dump, "scores_dump"), stream=stream)


def select_coverage_blocks(p: Problem, scores, qhat, khat, k_per_head, coverage: float, idx, cnt, rev_ptr, rev_idx,
                           workspace, scores_dump=None, stream=None) -> None:
    """Per row, the shortest run of blocks in score order whose estimated attention mass reaches coverage
    (at most k_h); counts to cnt [B, H, NG]."""
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_select_coverage_blocks", ctypes.byref(p.c()), a.scores(scores), a.qhat(qhat), a.khat(khat), kph,
           float(coverage), a.idx(idx, k_per_head), a.cnt(cnt), a.rev_ptr(rev_ptr),
           a.idx(rev_idx, k_per_head, "rev_idx"), a.scores(scores_dump, "scores_dump"), *a.ws(workspace),
           stream=stream)


def select_blocks(p: Problem, scores, qhat, khat, k_per_head, coverage: float, flags: int, idx, cnt, rev_ptr,
                  rev_idx, workspace, scores_dump=None, stream=None) -> None:
    """The general selection: top-k (coverage 0) or by coverage, optionally with the diagonal forced."""
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_select_blocks", ctypes.byref(p.c()), a.scores(scores), a.qhat(qhat), a.khat(khat), kph,
           float(coverage), int(flags), a.idx(idx, k_per_head), a.cnt(cnt, required=False), a.rev_ptr(rev_ptr),
           a.idx(rev_idx, k_per_head, "rev_idx"), a.scores(scores_dump, "scores_dump"), *a.ws(workspace),
           stream=stream)


def sparse_attn_fwd(p: Problem, Q, K, V, idx, k_per_head, O, LSE, workspace=None, stream=None) -> None:
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_sparse_attn_fwd", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"),
           a.idx(idx, k_per_head), kph, a.out(O, "O"), a.rows(LSE, "LSE"), *a.ws(workspace, False),
           stream=stream)


def sparse_attn_fwd_varlen(p: Problem, Q, K, V, idx, cnt, k_per_head, O, LSE, workspace=None, stream=None) -> None:
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_sparse_attn_fwd_varlen", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"),
           a.idx(idx, k_per_head), a.cnt(cnt), kph, a.out(O, "O"), a.rows(LSE, "LSE"), *a.ws(workspace, False),
           stream=stream)


def sparse_attn_fwd_split(p: Problem, Q, K, V, idx, k_per_head, n_split: int, O_part, LSE_part, workspace=None,
                          stream=None) -> None:
    """Partial states over n_split contiguous parts of every row's kept list: O_part [n_split, B, H, N, d],
    LSE_part [n_split, B, H, N] (fp32)."""
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    n = max(int(n_split), 1)
    a.call("dsa_sparse_attn_fwd_split", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"),
           a.idx(idx, k_per_head), kph, int(n_split), a.out(O_part, "O_part", n), a.rows(LSE_part, "LSE_part", n),
           *a.ws(workspace, False), stream=stream)


def attn_merge(p: Problem, n_parts: int, O_part, LSE_part, O, LSE, stream=None) -> None:
    """O, LSE from n_parts partial states (log-sum-exp weighted)."""
    a = _Args(p)
    n = max(int(n_parts), 1)
    a.call("dsa_attn_merge", ctypes.byref(p.c()), int(n_parts), a.out(O_part, "O_part", n),
           a.rows(LSE_part, "LSE_part", n), a.out(O, "O"), a.rows(LSE, "LSE"), stream=stream)


def dense_attn_fwd(p: Problem, Q, K, V, O, LSE, workspace=None, stream=None) -> None:
    """Full attention over every key (the dispatcher's dense branch)."""
    a = _Args(p)
    a.call("dsa_dense_attn_fwd", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"), a.out(O, "O"),
           a.rows(LSE, "LSE"), *a.ws(workspace, False), stream=stream)


def dense_attn_bwd(p: Problem, Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, stream=None) -> None:
    a = _Args(p)
    a.call("dsa_dense_attn_bwd", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"), a.out(O, "O"),
           a.io(dO, "dO"), a.rows(LSE, "LSE"), a.out(dQ, "dQ"), a.out(dK, "dK"), a.out(dV, "dV"), *a.ws(workspace),
           stream=stream)


def predictor_loss_grad(p: Problem, Q, K, Wq, Wk, loss, dWq, dWk, workspace, stream=None) -> None:
    """Stage-1 predictor training: loss [H] and its gradients dWq, dWk [H, d, r] (all fp32)."""
    a = _Args(p)
    a.call("dsa_predictor_loss_grad", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.weights(Wq, "Wq"),
           a.weights(Wk, "Wk"), a.f32(loss, "loss", p.heads), a.weights(dWq, "dWq"), a.weights(dWk, "dWk"),
           *a.ws(workspace), stream=stream)


def choose_path(p: Problem, k_per_head: Sequence[int], min_sparsity: float = -1.0, max_sparse_bytes: int = 0) -> int:
    """PATH_SPARSE or PATH_DENSE for one layer (min_sparsity < 0: the library's measured default)."""
    st = library().dsa_choose_path(ctypes.byref(p.c()), _kph(k_per_head, p.heads), float(min_sparsity),
                                   int(max_sparse_bytes))
    if st < 0:
        _check("dsa_choose_path", st)
    return st


def sparse_attn_bwd(p: Problem, Q, K, V, O, dO, LSE, idx, k_per_head, rev_ptr, rev_idx, dQ, dK, dV, workspace,
                    stream=None, flags: int = 0) -> None:
    """flags: BWD_V_FROM_FORWARD when ``workspace`` went to the forward of these inputs (V's copy reused)."""
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    args = [ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"), a.out(O, "O"), a.io(dO, "dO"),
            a.rows(LSE, "LSE"), a.idx(idx, k_per_head), kph, a.rev_ptr(rev_ptr), a.idx(rev_idx, k_per_head, "rev_idx"),
            a.out(dQ, "dQ"), a.out(dK, "dK"), a.out(dV, "dV")]
    if flags:
        a.call("dsa_sparse_attn_bwd_ex", *args, int(flags), *a.ws(workspace), stream=stream)
    else:
        a.call("dsa_sparse_attn_bwd", *args, *a.ws(workspace), stream=stream)


def sparse_attn_bwd_varlen(p: Problem, Q, K, V, O, dO, LSE, idx, cnt, k_per_head, rev_ptr, rev_idx, dQ, dK, dV,
                           workspace, stream=None) -> None:
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_sparse_attn_bwd_varlen", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"),
           a.out(O, "O"), a.io(dO, "dO"), a.rows(LSE, "LSE"), a.idx(idx, k_per_head), a.cnt(cnt), kph,
           a.rev_ptr(rev_ptr), a.idx(rev_idx, k_per_head, "rev_idx"), a.out(dQ, "dQ"), a.out(dK, "dK"),
           a.out(dV, "dV"), *a.ws(workspace), stream=stream)


def sparse_attn_bwd_preprocess(p: Problem, Q, K, V, O, dO, LSE, workspace, stream=None, flags: int = 0) -> None:
    a = _Args(p)
    args = [ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"), a.out(O, "O"), a.io(dO, "dO"),
            a.rows(LSE, "LSE")]
    if flags:
        a.call("dsa_sparse_attn_bwd_preprocess_ex", *args, int(flags), *a.ws(workspace), stream=stream)
    else:
        a.call("dsa_sparse_attn_bwd_preprocess", *args, *a.ws(workspace), stream=stream)


def sparse_attn_bwd_dkdv(p: Problem, Q, K, V, dO, k_per_head, rev_ptr, rev_idx, dK, dV, workspace,
                         stream=None) -> None:
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_sparse_attn_bwd_dkdv", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(K, "K"), a.io(V, "V"),
           a.io(dO, "dO"), kph, a.rev_ptr(rev_ptr), a.idx(rev_idx, k_per_head, "rev_idx"), a.out(dK, "dK"),
           a.out(dV, "dV"), *a.ws(workspace), stream=stream)


def sparse_attn_bwd_dq(p: Problem, Q, dO, idx, k_per_head, dQ, workspace, stream=None) -> None:
    a = _Args(p)
    kph = _kph(k_per_head, p.heads)
    a.call("dsa_sparse_attn_bwd_dq", ctypes.byref(p.c()), a.io(Q, "Q"), a.io(dO, "dO"), a.idx(idx, k_per_head), kph,
           a.out(dQ, "dQ"), *a.ws(workspace), stream=stream)


class SparseAttentionPlan:
    """Outputs and workspaces of one problem, allocated once with torch, plus the calls in order."""

    def __init__(self, p: Problem, k_per_head: Sequence[int], device="cuda", materialise_scores: bool = True,
                 backward: bool = True, coverage: Optional[float] = None, select_flags: int = 0,
                 reuse_v: bool = True):
        """coverage: select by attention coverage (k_per_head is then each row's capacity) and run the
        per-row-count forward and backward; select_flags: SELECT_DIAGONAL keeps each group's own blocks;
        reuse_v (training plans, bf16): the forward writes its scaled fp16 copy of V into the backward's
        workspace and the backward reuses it (BWD_V_FROM_FORWARD) instead of converting V again."""
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
        self.reuse_v = bool(reuse_v and backward and p.dtype == DSA_BF16 and coverage is None)
        if backward:
            self.dQ = torch.empty(B, H, N, D, **f32)
            self.dK = torch.empty(B, H, N, D, **f32)
            self.dV = torch.empty(B, H, N, D, **f32)
            self.ws_bwd = torch.empty(workspace_bytes(p, self.k_per_head, DSA_WS_BWD), dtype=torch.uint8,
                                      device=device)
            if self.reuse_v:
                self.ws_fwd = self.ws_bwd   # the forward's layout is the start of the backward's

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
                            self.rev_idx, self.dQ, self.dK, self.dV, self.ws_bwd, stream,
                            flags=BWD_V_FROM_FORWARD if self.reuse_v else 0)

    def backward_stages(self, Q, K, V, dO, stream=None):
        """The backward as its three stages (same result as backward()); top-k selection only."""
        if self.cnt is not None:
            raise ValueError("the staged backward takes no per-row counts: use backward()")
        sparse_attn_bwd_preprocess(self.p, Q, K, V, self.O, dO, self.LSE, self.ws_bwd, stream,
                                   flags=BWD_V_FROM_FORWARD if self.reuse_v else 0)
        sparse_attn_bwd_dkdv(self.p, Q, K, V, dO, self.k_per_head, self.rev_ptr, self.rev_idx, self.dK, self.dV,
                             self.ws_bwd, stream)
        sparse_attn_bwd_dq(self.p, Q, dO, self.idx, self.k_per_head, self.dQ, self.ws_bwd, stream)

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
