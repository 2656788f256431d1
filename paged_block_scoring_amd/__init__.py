"""Paged block scoring (QSA-style sparse-attention indexer) for MI355X.

The hot path -- score every causally visible compressed key of a paged side
cache against each query row's index heads, then keep the row's exact
lexicographic top-k blocks as token indices -- runs in hand-written gfx950
HIP kernels behind the C ABI of ``include/qsa.h``.  ``paged_block_scoring_amd.qsa``
is the thin ctypes binding.
"""
from .qsa import (  # noqa: F401
    QSA_MAX_SELECT, QSA_OUT_KEYS, QSA_SCORE_RELU, QSAError, qsa_last_error, qsa_last_path,
    qsa_score_paged, qsa_select_paged_tokens, qsa_select_paged_tokens_workspace_size, qsa_topk_rows,
    qsa_topk_rows_workspace_size, qsa_version,
)
