"""CPU oracle for the HISA and flat DSA indexers and the sparse attention after them -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path never calls it.
"""
from .oracle import (  # noqa: F401
    load,
    num_threads,
    score,
    mean_rows,
    max_rows,
    pool,
    super_pool,
    flat_query,
    refine_query,
    hisa_query,
    block_sparse_query,
    tree_query,
    tree_super_scores,
    hisa_batch,
    flat_batch,
    sparse_attention,
    sparse_attention_batch,
)
