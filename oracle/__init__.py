"""CPU oracle for Spatial Sparse Attention (SSA) over sparse-voxel tokens.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The
product path (``spatial_sparse_attention_ssa_amd``) never calls it, and shares
no code, headers, tables or helpers with it.

The oracle is a plain, slow, float64 numpy transcription of the method as the
Direct3D-S2 summary page states it (hyper.ai, arXiv 2505.17412, "Method",
second paragraph): tokens are blocked by 3D coordinate; keys and values are
mean-pooled per m_cmp^3 block; every query attends to the compressed blocks;
the query-to-block attention scores pick the top-k blocks, whose tokens take
part in a second attention; a third attention runs inside non-overlapping
m_win^3 windows; the three outputs are summed with predicted per-token gates.
Grouped-query sharing of the selection follows LSRM's 32-query / 2-KV-head
layout (LSRM article, "Stage 1").  The backward pass gives the gradients of
that output with respect to the queries, keys, values and gates, with the
top-k choice held fixed.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against closed
forms, library routines, brute force and hand-worked cases.
"""

from .ssa_oracle import (  # noqa: F401
    Blocks,
    bf16_round,
    block_keys,
    build_blocks,
    pool_blocks,
    softmax_attention,
    topk_blocks,
    geometric_topk,
    forward,
    forward_rows,
    backward,
    backward_rows,
    pooled_to_tokens,
    softmax_attention_grad,
    round_to,
)
