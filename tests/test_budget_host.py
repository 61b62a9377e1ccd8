"""The library's host tree-budget policy against ``oracle.budget`` (CPU only: these entry
points are host arithmetic and need no GPU).  Chosen paths and tree sizes bit-exact;
expected tokens to 1e-12 (both sides sum the same products in node order)."""
import numpy as np
import pytest

import tree_attention_draft_amd as tv
from oracle import budget as ob
from oracle import meta as om
from tree_attention_draft_amd import workloads


def random_probs(rng, k):
    w = rng.random(k + 1) ** 2
    return list(w[:k] / w.sum())


@pytest.mark.parametrize("seed", range(10))
def test_expected_tokens_random_trees(seed):
    rng = np.random.Generator(np.random.PCG64(4400 + seed))
    for n in (1, 2, 10, 33, 64):
        paths, _ = workloads.random_tree(rng, n, 8)
        b = om.build_from_paths(paths, 0)
        rank = [0] + [p[-1] for p in b["paths"][1:]]
        probs = random_probs(rng, int(rng.integers(1, 6)))
        e, reach = tv.tree_expected_tokens(b["parent"], rank, probs)
        assert abs(e - ob.expected_tokens(b["parent"], rank, probs)) < 1e-12
        assert np.array_equal(reach, np.array(ob.reach_probabilities(b["parent"], rank, probs)))


def test_ridge_and_nodes_grid():
    assert tv.tree_ridge_tokens(989e12, 3.35e12, 2) == ob.ridge_tokens(989e12, 3.35e12, 2)
    mi = tv.tree_ridge_tokens(2.5e15, 8e12, 2)
    assert mi == ob.ridge_tokens(2.5e15, 8e12, 2) == 312.5
    for ridge in (0.0, 1.0, 63.9, 64.0, 295.2238805970149, 312.5, 1e6):
        for batch in (1, 2, 3, 7, 16, 29, 30, 59, 60, 64, 128, 296, 313, 10**6):
            for cap in (1, 5, 33, 64):
                assert tv.tree_budget_nodes(batch, ridge, cap) == \
                    ob.nodes_for_batch(batch, ridge, cap), (batch, ridge, cap)


@pytest.mark.parametrize("seed", range(12))
def test_best_static_matches_oracle(seed):
    rng = np.random.Generator(np.random.PCG64(4500 + seed))
    k = int(rng.integers(1, 5))
    probs = random_probs(rng, k)
    if seed % 4 == 0:                   # equal probabilities: ties decided by the path rule
        probs = [0.3] * k if k <= 3 else [0.2] * k
    for nodes in (1, 2, 5, 10, 17, 33, 64):
        for depth in (1, 3, 6):
            if k ** depth > 5000:
                continue
            got, e = tv.tree_best_static(probs, nodes, depth)
            want = ob.best_static_tree(probs, nodes, depth)
            assert got == want, (probs, nodes, depth)
            pr, rk = ob_tree(want)
            assert abs(e - ob.expected_tokens(pr, rk, probs)) < 1e-12


def ob_tree(paths):
    b = om.build_from_paths(paths, 0)
    return b["parent"], [0] + [p[-1] for p in paths]


def test_page_figures_through_the_library():
    _, e10 = tv.tree_best_static([0.7, 0.15], 10, 4)
    assert abs(e10 - 3.2801) < 1e-12
    chain, e5 = tv.tree_best_static([0.7, 0.15], 5, 4)
    assert chain == [(0,), (0, 0), (0, 0, 0), (0, 0, 0, 0)] and abs(e5 - 2.7731) < 1e-12
    ridge = tv.tree_ridge_tokens(989e12, 3.35e12, 2)
    assert tv.tree_budget_nodes(29, ridge) >= 10 > tv.tree_budget_nodes(30, ridge)
    assert tv.tree_budget_nodes(59, ridge) >= 5 > tv.tree_budget_nodes(60, ridge)


def test_plan_matches_oracle_and_feeds_the_builder():
    ridge = tv.tree_ridge_tokens(2.5e15, 8e12, 2)
    probs = [0.62, 0.18, 0.07]
    for batch in (1, 4, 9, 16, 31, 64, 128, 313):
        n, paths, e = tv.tree_budget_plan(batch, ridge, probs, 64, 8)
        n_ref, paths_ref = ob.plan(batch, ridge, probs, 64, 8)
        assert (n, paths) == (n_ref, paths_ref)
        meta = tv.tree_meta_build(paths, 100)        # a valid tree for the builder
        assert len(meta["parent"]) == len(paths) + 1 <= n


def test_errors():
    with pytest.raises(tv.TreeVerifyError):
        tv.tree_expected_tokens([-1, 0, 0], [0, 1, 1], [0.5, 0.4])      # sibling ranks
    with pytest.raises(tv.TreeVerifyError):
        tv.tree_expected_tokens([-1, 1], [0, 0], [0.5])                 # parent order
    with pytest.raises(tv.TreeVerifyError):
        tv.tree_expected_tokens([-1, 0], [0, 0], [0.7, 0.5])            # sum above 1
    with pytest.raises(tv.TreeVerifyError):
        tv.tree_expected_tokens([-1, 0], [0, 0], [float("nan")])
    with pytest.raises(tv.TreeVerifyError):
        tv.tree_budget_nodes(0, 100.0)
    with pytest.raises(tv.TreeVerifyError):
        tv.tree_budget_nodes(4, float("inf"))
    with pytest.raises(tv.TreeVerifyError):
        tv.tree_ridge_tokens(0.0, 1.0)
    with pytest.raises(tv.TreeVerifyError) as ei:
        tv.tree_best_static([0.5], 65, 4)
    assert ei.value.name == "TV_ERR_CAPACITY"
    with pytest.raises(tv.TreeVerifyError):
        tv.tree_best_static([0.5], 10, 0)
