"""Tree-verification attention for MI355X (gfx950).

The work runs in ``libtreeverify.so`` (hand-written HIP kernels plus a host C++ tree
builder) behind the C ABI declared in ``include/tree_verify.h``; this package is its thin
Python binding plus the seeded workload generators used by the tests and the benchmark.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MAX_NODES, PackedTrees, PreparedAttn, PreparedBuild, PreparedCall,
    TreeVerifyError, TvAcceptArgs, TvAttnArgs, prepare_tree_accept_greedy,
    prepare_tree_accept_stochastic, prepare_tree_kv_compact, prepare_tree_meta_build_batch,
    prepare_tree_verify_attn,
    TvCompactArgs, TvSampleArgs, lib, make_accept_args, make_args, make_compact_args,
    make_sample_args, tree_accept_greedy, tree_accept_stochastic,
    tree_best_static, tree_budget_nodes, tree_budget_plan, tree_expected_tokens,
    tree_kv_compact, tree_meta_build, tree_meta_build_batch, tree_meta_from_parent,
    tree_ridge_tokens, tree_verify_attn, tree_verify_attn_static,
    tree_verify_attn_workspace_size, STATIC_SCRATCH_BYTES)
