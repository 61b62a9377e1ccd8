"""Pins for the tree-budget oracle (CPU only).

``oracle.budget`` is pinned against things other than itself:
* the figures [TAM] "What it buys" and "What it costs" print: 3.28 expected tokens for the
  worked tree and 2.77 for the chain of four at r0 = 0.7, r1 = 0.15 (gain 1.18x); a ridge of
  roughly 295 tokens from 989 TFLOP/s and 3.35 TB/s with two-byte weights; break-even
  batches of about 29 (tree) and 59 (chain); 640 and 320 tokens per step at batch 64, past
  the ridge by 2.2x;
* expected tokens by exact enumeration of every greedy outcome through the acceptance
  walk (``oracle.accept``), on random trees and probabilities;
* optimality of the best static tree by brute force over every ancestor-closed node set
  of small rank trees;
* the page's chain of four is the best 5-node tree and the worked tree's value is the best
  10-node value at depth <= 4;
* planted mistakes fail these pins.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import accept, budget, meta

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_tree.json")
PAGE_PROBS = [0.7, 0.15]


def ranked(paths):
    """(parent, rank) of the tree the builder makes from rank paths."""
    b = meta.build_from_paths(paths, 0)
    return b["parent"], [0] + [p[-1] for p in b["paths"][1:]]


def page_tree():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    return g, [tuple(p) for p in g["paths"]]


# ------------------------------------------------------------ the page's figures ----
def test_expected_tokens_of_the_page_trees():
    g, paths = page_tree()
    parent, rank = ranked(paths)
    e_tree = budget.expected_tokens(parent, rank, PAGE_PROBS)
    assert round(e_tree, 2) == g["expected_tokens_tree"] == 3.28
    assert abs(e_tree - 3.2801) < 1e-12
    chain = [(0,) * d for d in range(1, 5)]
    pc, rc = ranked(chain)
    e_chain = budget.expected_tokens(pc, rc, PAGE_PROBS)
    assert round(e_chain, 2) == g["expected_tokens_chain4"] == 2.77
    assert abs(e_chain - 2.7731) < 1e-12
    assert round(round(e_tree, 2) / round(e_chain, 2), 2) == 1.18


def test_reach_probabilities_are_the_printed_terms():
    _, paths = page_tree()
    parent, rank = ranked(paths)
    reach = budget.reach_probabilities(parent, rank, PAGE_PROBS)
    # level sums printed on the page: [0.7 + 0.15] [0.49 + 0.105 + 0.105]
    # [0.343 + 0.0735 + 0.0735] [0.2401]
    depth = meta.build_from_paths(paths, 0)["depth"]
    levels = {}
    for r, d in zip(reach, depth):
        levels.setdefault(d, []).append(r)
    assert sorted(levels[1]) == pytest.approx([0.15, 0.7], abs=1e-15)
    assert sorted(levels[2]) == pytest.approx([0.105, 0.105, 0.49], abs=1e-15)
    assert sorted(levels[3]) == pytest.approx([0.0735, 0.0735, 0.343], abs=1e-15)
    assert levels[4] == pytest.approx([0.2401], abs=1e-15)
    assert reach[0] == 1.0


def test_ridge_and_break_even_batches():
    ridge = budget.ridge_tokens(989e12, 3.35e12, 2)
    assert round(ridge) == 295
    # the page divides the rounded ridge; both readings give the same break-even batches
    for rg in (ridge, 295.0):
        assert budget.nodes_for_batch(29, rg, 64) >= 10 > budget.nodes_for_batch(30, rg, 64)
        assert budget.nodes_for_batch(59, rg, 64) >= 5 > budget.nodes_for_batch(60, rg, 64)
    # batch 64: 640 and 320 tokens per step, both past the ridge, the tree by 2.2x
    assert 64 * 10 == 640 and 64 * 5 == 320 and 320 > ridge
    assert round(640 / ridge, 1) == 2.2
    assert budget.nodes_for_batch(64, ridge, 64) == 4
    assert budget.nodes_for_batch(1, ridge, 64) == 64
    assert budget.nodes_for_batch(296, ridge, 64) == 1      # past the ridge: root only


# ------------------------------------------- independent: enumeration through the walk ----
def expected_by_enumeration(parent, rank, probs):
    """E[tokens emitted] over every greedy outcome: at each internal node the target's
    greedy token is the rank-r candidate with probability probs[r], else a token no child
    carries.  Draft token of a node = its rank."""
    n = len(parent)
    internal = sorted({p for p in parent if p >= 0})
    outcomes = [(r, p) for r, p in enumerate(probs)] + [(10**6, 1.0 - sum(probs))]
    total = 0.0
    for choice in itertools.product(outcomes, repeat=len(internal)):
        am = [10**6] * n
        pr = 1.0
        for node, (r, p) in zip(internal, choice):
            am[node] = r
            pr *= p
        _, emitted = accept.accept_greedy(parent, [-1] + list(rank[1:]), am)
        total += pr * len(emitted)
    return total


@pytest.mark.parametrize("seed", range(8))
def test_expected_tokens_equal_exact_enumeration(seed):
    rng = np.random.Generator(np.random.PCG64(900 + seed))
    k = int(rng.integers(1, 4))
    w = rng.random(k + 1)
    probs = list(w[:k] / w.sum())
    # random rank trees small enough to enumerate (at most 5 internal nodes)
    paths = set()
    while len(paths) < int(rng.integers(1, 8)):
        d = int(rng.integers(1, 4))
        p = tuple(int(x) for x in rng.integers(0, k + 1, size=d))
        for j in range(1, d + 1):
            paths.add(p[:j])
    parent, rank = ranked(sorted(paths))
    if len({p for p in parent if p >= 0}) > 5:
        pytest.skip("too many internal nodes to enumerate")
    got = budget.expected_tokens(parent, rank, probs)
    assert abs(got - expected_by_enumeration(parent, rank, probs)) < 1e-12


# --------------------------------------------------- optimality by brute force ------------
def brute_best_value(probs, nodes, max_depth):
    cands = [p for d in range(1, max_depth + 1)
             for p in itertools.product(range(len(probs)), repeat=d)]
    best = 1.0
    for k in range(0, min(nodes - 1, len(cands)) + 1):
        for sub in itertools.combinations(cands, k):
            s = set(sub)
            if all(p[:-1] in s or len(p) == 1 for p in sub):
                best = max(best, 1.0 + sum(budget.path_product(p, probs) for p in sub))
    return best


@pytest.mark.parametrize("probs,depth", [([0.6, 0.3], 3), ([0.5, 0.25, 0.2], 2),
                                         ([0.45, 0.45], 3), ([0.9], 4)])
@pytest.mark.parametrize("nodes", [1, 2, 4, 6, 8])
def test_best_static_tree_is_optimal(probs, depth, nodes):
    paths = budget.best_static_tree(probs, nodes, depth)
    assert len(paths) <= nodes - 1
    assert all(len(p) <= depth for p in paths)
    parent, rank = ranked(paths)                      # builder accepts it: ancestor-closed
    value = budget.expected_tokens(parent, rank, probs)
    assert abs(value - brute_best_value(probs, nodes, depth)) < 1e-12


def test_page_chain_is_the_best_five_node_tree():
    assert budget.best_static_tree(PAGE_PROBS, 5, 4) == [(0,), (0, 0), (0, 0, 0), (0, 0, 0, 0)]


def test_page_tree_value_is_the_best_ten_node_value():
    paths = budget.best_static_tree(PAGE_PROBS, 10, 4)
    assert len(paths) == 9
    parent, rank = ranked(paths)
    assert abs(budget.expected_tokens(parent, rank, PAGE_PROBS) - 3.2801) < 1e-12
    assert {(0,), (1,), (0, 0), (0, 1), (1, 0), (0, 0, 0), (0, 0, 0, 0)} <= set(paths)


def test_zero_probability_paths_are_never_taken():
    paths = budget.best_static_tree([1.0, 0.0], 8, 3)
    assert paths == [(0,), (0, 0), (0, 0, 0)]


def test_plan_shrinks_toward_a_chain():
    ridge = budget.ridge_tokens(989e12, 3.35e12, 2)
    sizes = []
    for b in (1, 8, 16, 29, 40, 59, 100, 300):
        n, paths = budget.plan(b, ridge, PAGE_PROBS, 64, 8)
        assert len(paths) == n - 1
        sizes.append(n)
    assert sizes == sorted(sizes, reverse=True) and sizes[-1] == 1
    n, paths = budget.plan(59, ridge, PAGE_PROBS, 64, 8)
    assert paths == [(0,) * d for d in range(1, 5)]        # a chain of four


def test_invalid_inputs_rejected():
    with pytest.raises(ValueError):
        budget.expected_tokens([-1, 0, 0], [0, 1, 1], PAGE_PROBS)      # equal sibling ranks
    with pytest.raises(ValueError):
        budget.expected_tokens([-1, 0], [0, 0], [0.7, 0.5])            # sum above 1
    with pytest.raises(ValueError):
        budget.nodes_for_batch(0, 295.0, 64)


# ------------------------------------------------------------------- planted -------------
def test_planted_mistakes_fail():
    _, paths = page_tree()
    parent, rank = ranked(paths)

    def no_root(parent, rank, probs):                  # forgets the root's token
        return sum(budget.reach_probabilities(parent, rank, probs)[1:])

    def ascending(probs, nodes, depth):                # keeps the least likely paths
        c = [(budget.path_product(p, probs), len(p), p) for d in range(1, depth + 1)
             for p in itertools.product(range(len(probs)), repeat=d)]
        return sorted(x[2] for x in sorted(c)[:nodes - 1])

    def ceil_nodes(batch, ridge, max_nodes):          # rounds the budget up
        return max(1, min(max_nodes, -(-int(ridge) // batch)))

    assert abs(no_root(parent, rank, PAGE_PROBS) - 3.2801) > 0.5
    bad = ascending([0.6, 0.3], 4, 3)
    assert len({p[:-1] for p in bad if len(p) > 1} - set(bad)) > 0      # not even a tree
    assert ceil_nodes(30, 295.0, 64) == 10 != budget.nodes_for_batch(30, 295.0, 64)
