"""float64 CPU oracle of the DSV sparse-attention hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the bench's CPU-baseline leg
may import this package.  The product (the HIP library and its binding) never
does, and the two implementations share no code; they meet only in the seeded
inputs drawn by the ``synth`` package.

Every function is pinned by tests/test_oracle.py (brute force, a library
routine, finite differences, closed forms, invariants); none is "parity
unpinned".
"""
from . import dsv_oracle
from .dsv_oracle import (
    BLOCK, backward, backward_head, dense_backward, dense_backward_head, dense_dkdv_blocks, dense_dq_rows,
    dense_forward, dense_forward_head, dense_rows, dkdv_blocks, dq_groups, forward, forward_head,
    forward_split_head, group_backward, group_forward, kept_keys, merge_states, partial_state, pool_mean, predict,
    predict_head, predictor_loss_grad, predictor_loss_grad_head, predictor_loss_head, reverse_index, reverse_list,
    select, select_row, sparsity, split_bounds, use_sparse, block_mass, select_coverage_row, select_coverage,
    diagonal_blocks, select_order, select_row_diag, select_coverage_row_diag, predict_head_pooled,
    predict_head_pooled_groups, predict_head_pooled_rows, select_rows, reverse_index_csr, dkdv_block_part,
)

__all__ = [
    "dsv_oracle", "BLOCK", "backward", "backward_head", "dense_backward", "dense_backward_head",
    "dense_dkdv_blocks", "dense_dq_rows", "dense_forward", "dense_forward_head", "dense_rows", "sparsity",
    "use_sparse", "block_mass", "select_coverage_row", "select_coverage", "diagonal_blocks", "select_order",
    "select_row_diag", "select_coverage_row_diag", "predict_head_pooled",
    "predict_head_pooled_groups", "predict_head_pooled_rows", "predictor_loss_head", "predictor_loss_grad_head", "predictor_loss_grad", "dkdv_blocks",
    "dq_groups", "forward",
    "forward_head", "forward_split_head", "group_backward", "group_forward", "kept_keys", "merge_states",
    "partial_state", "pool_mean", "predict", "predict_head", "reverse_index", "reverse_list", "select",
    "select_row", "split_bounds", "select_rows", "reverse_index_csr", "dkdv_block_part",
]
