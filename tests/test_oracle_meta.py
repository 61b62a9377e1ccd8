"""Pins for the oracle's tree metadata (CPU only).

Each pin is checked against something other than the oracle's own code: values printed on
"Tree attention mask for draft-tree verification" (worked example, empty tree, missing
parent), the page's expected-token arithmetic, and an independent derivation of the
ancestor relation as the reflexive-transitive closure of the child->parent edge relation.
"""
import itertools
import json
import os
import random

import numpy as np
import pytest

from oracle import meta
from tree_attention_draft_amd import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "worked_example_tree.json")))
TEN_PARENT = [-1, 0, 0, 1, 1, 2, 3, 3, 4, 6]     # the 10-node workload's stated tree
TEN_DEPTH = [0, 1, 1, 2, 2, 2, 3, 3, 3, 4]


def all_parent_arrays(n):
    """Every parent-before-child labelled tree with n nodes."""
    ranges = [range(i) for i in range(1, n)]
    for choice in itertools.product(*ranges):
        yield [-1] + list(choice)


def closure_mask(parent):
    """Ancestor-or-self relation as the reflexive-transitive closure of child->parent."""
    n = len(parent)
    E = np.zeros((n, n), dtype=np.int64)
    for i, p in enumerate(parent):
        if p >= 0:
            E[i, p] = 1
    R = np.eye(n, dtype=np.int64)
    step = np.eye(n, dtype=np.int64)
    for _ in range(n):
        step = (step @ E > 0).astype(np.int64)
        R = ((R + step) > 0).astype(np.int64)
    return R.astype(bool)


def expected_tokens(paths, rank_prob):
    total = 1.0
    for p in paths:
        prod = 1.0
        for r in p:
            prod *= rank_prob[r]
        total += prod
    return total


# ------------------------------------------------------------------ worked example ----
def test_worked_example_printed_rows():
    t = meta.build_from_paths([tuple(p) for p in GOLD["paths"]], GOLD["prefix_len"])
    for row, cols in GOLD["printed_mask_rows"].items():
        got = [j for j, ok in enumerate(t["mask"][int(row)]) if ok]
        assert got == cols
        assert t["bitmask"][int(row)] == sum(1 << j for j in cols)


def test_worked_example_structure_matches_workload_tree():
    t = meta.build_from_paths([tuple(p) for p in GOLD["paths"]], GOLD["prefix_len"])
    assert t["parent"] == TEN_PARENT
    assert t["depth"] == TEN_DEPTH
    assert t["pos"] == [GOLD["prefix_len"] + d for d in TEN_DEPTH]
    a, b = GOLD["siblings_share_position"]
    assert t["pos"][a] == t["pos"][b]
    assert [hex(m) for m in t["bitmask"]] == [
        "0x1", "0x3", "0x5", "0xb", "0x13", "0x25", "0x4b", "0x8b", "0x113", "0x24b"]


def test_worked_example_expected_tokens():
    r = {int(k): v for k, v in GOLD["rank_acceptance"].items()}
    paths = [tuple(p) for p in GOLD["paths"]]
    e_tree = expected_tokens(paths, r)
    e_chain = expected_tokens(workloads.chain_paths(5), r)
    assert round(e_tree, 2) == GOLD["expected_tokens_tree"]
    assert round(e_chain, 2) == GOLD["expected_tokens_chain4"]
    assert round(e_tree / e_chain, 2) == GOLD["gain"]
    assert len(paths) + 1 == GOLD["verified_tokens_tree"]
    # the level-by-level terms printed on the page
    t = meta.build_from_paths(paths, 0)
    by_level = {}
    for p in t["paths"][1:]:
        prod = 1.0
        for x in p:
            prod *= r[x]
        by_level.setdefault(len(p), []).append(prod)
    for lvl, terms in enumerate(GOLD["expected_tokens_tree_level_terms"], start=1):
        assert sorted(round(x, 4) for x in by_level[lvl]) == sorted(terms)


def test_workload_module_holds_the_same_tree():
    assert [list(p) for p in workloads.TEN_NODE_PATHS] == GOLD["paths"]


def test_chain_structure():
    t = meta.build_from_paths(workloads.chain_paths(5), 7)
    assert t["parent"] == [-1, 0, 1, 2, 3]
    assert [hex(m) for m in t["bitmask"]] == ["0x1", "0x3", "0x7", "0xf", "0x1f"]
    assert t["pos"] == [7, 8, 9, 10, 11]


# ------------------------------------------------------------------ special cases -----
def test_empty_tree_is_plain_decoding():
    t = meta.build_from_paths([], 123)
    assert t["parent"] == [-1] and t["depth"] == [0] and t["pos"] == [123]
    assert t["mask"] == [[True]]
    assert t["bitmask"] == [1]


@pytest.mark.parametrize("paths,bad", [([(0, 0)], 0), ([(1,), (0, 1)], 1),
                                       ([(0,), (2, 0), (0, 0)], 1),
                                       ([(0,), (0, 0, 0)], 1)])
def test_missing_parent_is_rejected(paths, bad):
    with pytest.raises(meta.TreeError) as e:
        meta.build_from_paths(paths, 0)
    assert e.value.code == "missing_parent"
    assert e.value.index == bad


@pytest.mark.parametrize("paths,bad", [([(0,), ()], 1), ([(0,), (0, -1)], 1)])
def test_invalid_paths_are_rejected(paths, bad):
    with pytest.raises(meta.TreeError) as e:
        meta.build_from_paths(paths, 0)
    assert e.value.code == "invalid_path" and e.value.index == bad


def test_capacity():
    paths = [(i,) for i in range(63)]
    assert len(meta.build_from_paths(paths, 0)["parent"]) == 64
    with pytest.raises(meta.TreeError) as e:
        meta.build_from_paths(paths + [(63,)], 0)
    assert e.value.code == "capacity"


def test_duplicates_collapse_and_input_order_is_irrelevant():
    rng = random.Random(5)
    base = [tuple(p) for p in GOLD["paths"]]
    ref = meta.build_from_paths(base, 3)
    for _ in range(20):
        shuffled = base + rng.sample(base, 4)
        rng.shuffle(shuffled)
        t = meta.build_from_paths(shuffled, 3)
        for key in ("parent", "depth", "pos", "bitmask", "paths"):
            assert t[key] == ref[key]


# --------------------------------------------------- independent derivation sweeps ---
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_mask_is_ancestor_closure_all_small_trees(n):
    count = 0
    for parent in all_parent_arrays(n):
        m = meta.meta_from_parent(parent, 11)
        R = closure_mask(parent)
        assert np.array_equal(np.array(m["mask"], dtype=bool), R)
        for i in range(n):
            assert m["bitmask"][i] == sum(1 << j for j in range(n) if R[i, j])
            assert m["depth"][i] == int(R[i].sum()) - 1
            assert m["pos"][i] == 11 + m["depth"][i]
        count += 1
    assert count == [1, 1, 2, 6, 24, 120][n - 1]


def test_paths_and_parent_forms_agree_on_random_trees():
    rng = np.random.Generator(np.random.PCG64(77))
    for n, cap in [(33, 8), (64, 10), (17, 3), (2, 1)]:
        for _ in range(10):
            paths, creation = workloads.random_tree(rng, n, cap)
            t = meta.build_from_paths(paths, 5)
            f = meta.meta_from_parent(t["parent"], 5)
            for key in ("depth", "pos", "bitmask", "mask"):
                assert t[key] == f[key]
            assert max(t["depth"]) <= cap
            # depth-sorted canonical order; every node's path extends its parent's
            assert t["depth"] == sorted(t["depth"])
            for i in range(1, n):
                assert t["paths"][i][:-1] == t["paths"][t["parent"][i]]
            # the generator's own creation order is a valid relabelling of the same tree
            g = meta.meta_from_parent(creation, 5)
            assert sorted(g["depth"]) == t["depth"]


@pytest.mark.parametrize("bad", [[0], [-1, 1], [-1, 0, 2], [-1, 0, -1], [-1, 5], []])
def test_invalid_parent_arrays_rejected(bad):
    with pytest.raises(meta.TreeError):
        meta.meta_from_parent(bad, 0)
