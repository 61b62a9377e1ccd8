"""Pins for the acceptance and compaction oracle (CPU only).

``oracle.accept`` is pinned against things other than itself:
* the walks the worked example's tests name ([TAM] "A strong answer"): one that takes the
  second-rank branch (it accepts nodes 0, 2, 5 -- the nodes [TAM] "What it costs" then
  compacts), one that goes down to the deepest leaf (four accepted drafts, then the
  bonus), the empty tree (one token) and a rejection at the root (one correction token);
* ``is_root_path`` against hand-made lists that break each of its conditions;
* the expected tokens per step the page prints (3.28 for the tree, 2.77 for the chain of
  four), recomputed by exact enumeration of every greedy outcome of the rank-acceptance
  model through the walk;
* an independent per-node characterisation of the accepted path (a node is on it iff its
  parent is, its token is the parent's greedy token, and no earlier sibling carries that
  token) on random trees and token draws;
* compaction: the page's example (nodes 0, 2, 5 to consecutive rows), untouched rows, and
  the defining property -- after compaction, ordinary causal attention at the last
  accepted position over the compacted cache equals the tree pass's output for that node;
* planted mistakes in copies of the walk must fail these pins.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import accept, attn, meta

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_tree.json")


def tree10():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    paths = [tuple(p) for p in g["paths"]]
    b = meta.build_from_paths(paths, g["prefix_len"])
    return g, paths, b["parent"]


def rank_tokens(paths):
    """Draft token of each node = its rank among its siblings (node 0: unused -1)."""
    return [-1] + [p[-1] for p in meta.build_from_paths(paths, 0)["paths"][1:]]


# ------------------------------------------------------------- the page's walks -----
def test_second_rank_branch_walk():
    _, paths, parent = tree10()
    tok = rank_tokens(paths)          # node 1 = (0,) rank 0, node 2 = (1,) rank 1, ...
    # target picks rank 1 at the root, rank 0 under node 2, then 7 at the leaf (bonus)
    am = [1, 9, 0, 9, 9, 7, 9, 9, 9, 9]
    acc, emitted = accept.accept_greedy(parent, tok, am)
    assert acc == [0, 2, 5]
    assert emitted == [1, 0, 7]       # two accepted drafts (ranks 1, 0) + the bonus


def test_deepest_leaf_walk_emits_four_drafts_and_bonus():
    _, paths, parent = tree10()
    tok = rank_tokens(paths)
    am = [0, 0, 9, 0, 9, 9, 0, 9, 9, 5]  # rank 0 all the way down 0 -> 1 -> 3 -> 6 -> 9
    acc, emitted = accept.accept_greedy(parent, tok, am)
    assert acc == [0, 1, 3, 6, 9]
    assert emitted == [0, 0, 0, 0, 5] and len(emitted) == 5


def test_empty_tree_emits_one_token():
    acc, emitted = accept.accept_greedy([-1], [-1], [42])
    assert acc == [0] and emitted == [42]


def test_rejection_at_root_emits_correction_only():
    _, paths, parent = tree10()
    tok = rank_tokens(paths)
    acc, emitted = accept.accept_greedy(parent, tok, [5] * 10)
    assert acc == [0] and emitted == [5]


def test_first_matching_sibling_wins():
    # two children carry the same token: the earlier one (node order) is taken
    acc, emitted = accept.accept_greedy([-1, 0, 0], [-1, 4, 4], [4, 8, 9])
    assert acc == [0, 1] and emitted == [4, 8]


# ------------------------------------------------------ expected tokens per step ----
def expected_tokens(parent, tok, probs):
    """E[len(emitted)] by exact enumeration: at every node the target's greedy token is
    rank r with probability probs[r], else (remaining mass) a token no child carries."""
    n = len(parent)
    outcomes = list(probs.items()) + [(99, 1.0 - sum(probs.values()))]
    total = 0.0
    for choice in itertools.product(outcomes, repeat=n):
        pr = float(np.prod([c[1] for c in choice]))
        am = [c[0] for c in choice]
        _, emitted = accept.accept_greedy(parent, tok, am)
        total += pr * len(emitted)
    return total


def test_expected_tokens_match_the_page():
    g, paths, parent = tree10()
    probs = {int(k): v for k, v in g["rank_acceptance"].items()}
    # enumerate only over the 6 internal nodes' outcomes (leaves emit a token whatever
    # the target picks): split the enumeration to keep it small
    internal = sorted({p for p in parent if p >= 0})
    tok = rank_tokens(paths)
    n = len(parent)
    outcomes = list(probs.items()) + [(99, 1.0 - sum(probs.values()))]
    total = 0.0
    for choice in itertools.product(outcomes, repeat=len(internal)):
        am = [99] * n
        pr = 1.0
        for node, (r, p) in zip(internal, choice):
            am[node] = r
            pr *= p
        _, emitted = accept.accept_greedy(parent, tok, am)
        total += pr * len(emitted)
    assert round(total, 2) == g["expected_tokens_tree"]
    assert abs(total - 3.2801) < 1e-12
    chain = [-1, 0, 1, 2, 3]
    ec = expected_tokens(chain, [-1, 0, 0, 0, 0], probs)
    assert round(ec, 2) == g["expected_tokens_chain4"]
    assert abs(ec - 2.7731) < 1e-12


# ------------------------------------------- independent characterisation -----------
def accepted_by_rule(parent, tok, am):
    n = len(parent)
    on = [False] * n
    on[0] = True
    for v in range(1, n):
        u = parent[v]
        earlier = any(parent[s] == u and tok[s] == am[u] for s in range(1, v))
        on[v] = on[u] and tok[v] == am[u] and not earlier
    acc = [v for v in range(n) if on[v]]
    return acc, [int(am[v]) for v in acc]


@pytest.mark.parametrize("seed", range(12))
def test_walk_matches_per_node_rule(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    from tree_attention_draft_amd import workloads
    for n in (1, 2, 5, 17, 33, 64):
        paths, _ = workloads.random_tree(rng, n, 8)
        parent = meta.build_from_paths(paths, 0)["parent"]
        vocab = int(rng.integers(2, 5))              # small vocabularies force matches
        tok = [-1] + list(rng.integers(0, vocab, size=len(parent) - 1))
        am = list(rng.integers(0, vocab, size=len(parent)))
        got = accept.accept_greedy(parent, tok, am)
        assert got == accepted_by_rule(parent, tok, am)
        assert accept.is_root_path(parent, got[0])


@pytest.mark.parametrize("lst,ok", [
    ([0], True), ([0, 2, 5], True), ([0, 1, 3, 6, 9], True),
    ([], False),                    # empty
    ([2, 5], False),                # does not start at the root
    ([1], False),                   # a single entry that is not the root
    ([0, 3], False),                # 3 is a grandchild of the root, not a child
    ([0, 1, 2], False),             # 2 is 1's sibling, not its child
    ([0, 10], False),               # out of range (N = 10)
    ([0, -1], False),               # negative entry
    ([0, 1, 3, 6, 9, 9], False),    # repeats the leaf: not a child of itself
    ([0, 2, 5, 5, 5, 5, 5, 5, 5, 5, 5], False),  # longer than N
    ([0, 0], False),                # the root again
])
def test_is_root_path_against_hand_made_lists(lst, ok):
    _, _, parent = tree10()         # parent = -1,0,0,1,1,2,3,3,4,6
    assert accept.is_root_path(parent, lst) is ok


def test_argmax_rows_ties_and_nan():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [np.nan, 5.0, np.nan, 1.0], [-1.0, -1.0, -1.0, -1.0]])
    assert accept.argmax_rows(x).tolist() == [1, 0, 0]


# ------------------------------------------------------------------- planted -------
def test_planted_mistakes_fail():
    _, paths, parent = tree10()
    tok = rank_tokens(paths)
    am = [1, 9, 0, 9, 9, 7, 9, 9, 9, 9]

    def walk_last_match(parent, tokens, target):     # takes the LAST matching child
        table = accept.child_table(parent)
        acc, em = [0], []
        for _ in range(len(parent)):
            em.append(target[acc[-1]])
            hit = [c for c in table[acc[-1]] if tokens[c] == target[acc[-1]]]
            if not hit:
                break
            acc.append(hit[-1])
        return acc, em

    def walk_no_bonus(parent, tokens, target):       # forgets the final token
        acc, em = accept.accept_greedy(parent, tokens, target)
        return acc, em[:-1]

    ref = accept.accept_greedy(parent, tok, am)
    assert walk_no_bonus(parent, tok, am) != ref
    assert walk_last_match([-1, 0, 0], [-1, 4, 4], [4, 8, 9]) != \
        accept.accept_greedy([-1, 0, 0], [-1, 4, 4], [4, 8, 9])


# ------------------------------------------------------------------ compaction ------
def test_compaction_of_the_page_example():
    rng = np.random.Generator(np.random.PCG64(7))
    L, n = 16, 10
    k = rng.standard_normal((L + n, 2, 8))
    v = rng.standard_normal((L + n, 2, 8))
    k2, v2, new_len = accept.compact_request(k, v, L, [0, 2, 5])
    assert new_len == L + 3
    for j, a in enumerate([0, 2, 5]):
        assert np.array_equal(k2[L + j], k[L + a]) and np.array_equal(v2[L + j], v[L + a])
    untouched = [t for t in range(L + n) if not (L <= t < L + 3)]
    assert np.array_equal(k2[untouched], k[untouched])
    assert np.array_equal(v2[untouched], v[untouched])


@pytest.mark.parametrize("seed", range(6))
def test_compacted_cache_reproduces_the_tree_output(seed):
    """After compaction, plain causal attention of the last accepted node's query over
    the first L + A rows equals the tree pass's output for that node ([TV] "Tree
    Attention": the pass computes exactly the conditional over the node's root path)."""
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    from tree_attention_draft_amd import workloads
    L, hq, hkv, d = int(rng.integers(0, 40)), 4, 2, 16
    paths, _ = workloads.random_tree(rng, 12, 5)
    parent = meta.build_from_paths(paths, L)["parent"]
    n = len(parent)
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((L + n, hkv, d))
    v = rng.standard_normal((L + n, hkv, d))
    out, lse = attn.tree_attention_request(q, k, v, parent, L)
    tok = [-1] + list(rng.integers(0, 2, size=n - 1))
    am = list(rng.integers(0, 2, size=n))
    acc, _ = accept.accept_greedy(parent, tok, am)
    k2, v2, new_len = accept.compact_request(k, v, L, acc)
    last = acc[-1]
    g = hq // hkv
    for h in range(hq):
        kk, vv = k2[:new_len, h // g], v2[:new_len, h // g]
        s = kk @ q[last, h] / np.sqrt(d)
        m = s.max()
        w = np.exp(s - m)
        ref = (w[:, None] * vv).sum(0) / w.sum()
        assert np.abs(ref - out[last, h]).max() < 1e-12
        assert abs(m + np.log(w.sum()) - lse[last, h]) < 1e-12
