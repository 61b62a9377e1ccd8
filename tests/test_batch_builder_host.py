"""The batched host builder ``tree_meta_build_batch`` against the oracle (CPU only).

Every row of the batched call must equal what ``oracle.meta.build_from_paths`` gives for
that request's candidates ("Tree attention mask for draft-tree verification", "A strong
answer": node order, parent, depth, ancestor mask, position = prefix + depth), trees
smaller than the row width are padded with leaves under the root, and a rejected tree
(missing parent, invalid path, too many nodes) is named by its batch index and the
offending candidate's index within it.
"""
import ctypes

import numpy as np
import pytest

import tree_attention_draft_amd as tv
from oracle import meta
from tree_attention_draft_amd import workloads
from tree_attention_draft_amd._binding import PackedTrees, TreeVerifyError


def check_rows(trees, L, N, got):
    for b, paths in enumerate(trees):
        ref = meta.build_from_paths(paths, int(L[b]))
        n = len(ref["parent"])
        assert got["num_nodes"][b] == n
        assert got["parent"][b, :n].tolist() == ref["parent"]
        assert got["depth"][b, :n].tolist() == ref["depth"]
        assert got["pos"][b, :n].tolist() == ref["pos"]
        assert [int(x) for x in got["bitmask"][b, :n]] == ref["bitmask"]
        # padding rows: extra leaves under the root, so the row is still a valid tree
        for i in range(n, N):
            assert got["parent"][b, i] == 0 and got["depth"][b, i] == 1
            assert got["pos"][b, i] == L[b] + 1
            assert int(got["bitmask"][b, i]) == (1 | (1 << i))
        meta.validate_parent(got["parent"][b].tolist())


def test_mixed_sizes_with_padding_rows():
    rng = np.random.Generator(np.random.PCG64(71))
    trees = [list(workloads.TEN_NODE_PATHS), [], workloads.chain_paths(5)]
    for n in (33, 2, 64, 17, 1):
        trees.append(workloads.random_tree(rng, n, 8)[0])
    L = np.array([16, 0, 7, 4096, 3, 32768, 511, 1], np.int32)
    got = tv.tree_meta_build_batch(PackedTrees(trees), L, 64)
    check_rows(trees, L, 64, got)


def test_equal_sizes_no_padding_and_workload_batch():
    spec = workloads.WORKLOADS["b64_l4096_n33"]
    trees, _ = workloads.trees_for(spec)
    L = workloads.prefix_lengths(spec)
    got = tv.tree_meta_build_batch(PackedTrees(trees), L, 33)
    check_rows(trees, L, 33, got)
    assert (got["num_nodes"] == 33).all()


def test_every_tree_empty():
    trees = [[] for _ in range(5)]
    L = np.arange(5, dtype=np.int32) * 10
    got = tv.tree_meta_build_batch(PackedTrees(trees), L, 3)
    check_rows(trees, L, 3, got)
    assert (got["num_nodes"] == 1).all()


@pytest.mark.parametrize("bad,code,bad_path", [
    ([(0,), (1, 0), (0, 0)], "TV_ERR_MISSING_PARENT", 1),   # (1,) missing
    ([(0,), (0, -2)], "TV_ERR_INVALID_PATH", 1),            # negative rank
    ([(0,), ()], "TV_ERR_INVALID_PATH", 1),                 # empty candidate
])
def test_failing_tree_in_the_middle_is_named(bad, code, bad_path):
    good = list(workloads.TEN_NODE_PATHS)
    trees = [good, good, bad, good]
    with pytest.raises(TreeVerifyError) as e:
        tv.tree_meta_build_batch(PackedTrees(trees), np.zeros(4, np.int32), 16)
    assert e.value.name == code
    assert e.value.bad_tree == 2 and e.value.bad_path == bad_path
    # the oracle rejects the same candidate of that tree
    with pytest.raises(meta.TreeError) as r:
        meta.build_from_paths(bad, 0)
    assert r.value.index == bad_path


def test_capacity_of_the_row_width():
    trees = [workloads.chain_paths(5), list(workloads.TEN_NODE_PATHS)]
    with pytest.raises(TreeVerifyError) as e:
        tv.tree_meta_build_batch(PackedTrees(trees), np.zeros(2, np.int32), 9)
    assert e.value.name == "TV_ERR_CAPACITY" and e.value.bad_tree == 1
    got = tv.tree_meta_build_batch(PackedTrees(trees), np.zeros(2, np.int32), 10)
    check_rows(trees, np.zeros(2, np.int32), 10, got)


def call_raw(ranks, path_off, tree_off, B, L, N, out_fill=-7):
    """Direct C call with caller-made CSR arrays; outputs pre-filled to detect writes."""
    par = np.full((max(B, 1), N), out_fill, np.int32)
    dep = np.full((max(B, 1), N), out_fill, np.int32)
    pos = np.full((max(B, 1), N), out_fill, np.int32)
    bm = np.full((max(B, 1), N), 7, np.uint64)
    nn = np.full(max(B, 1), out_fill, np.int32)
    bt, bp = ctypes.c_int32(99), ctypes.c_int32(99)
    st = tv.lib().tree_meta_build_batch(
        ranks.ctypes.data, path_off.ctypes.data, tree_off.ctypes.data, B, L.ctypes.data, N,
        par.ctypes.data, dep.ctypes.data, bm.ctypes.data, pos.ctypes.data, nn.ctypes.data,
        ctypes.byref(bt), ctypes.byref(bp))
    untouched = ((par == out_fill).all() and (dep == out_fill).all() and
                 (pos == out_fill).all() and (bm == 7).all() and (nn == out_fill).all())
    return st, bt.value, bp.value, untouched


def test_argument_errors_write_nothing():
    ranks = np.array([0, 0, 0, 1, 0], np.int32)
    path_off = np.array([0, 1, 3, 4, 5], np.int64)       # (0,), (0,0), (1,), (0,)
    L = np.zeros(2, np.int32)
    ok = np.array([0, 3, 4], np.int64)
    st, bt, bp, untouched = call_raw(ranks, path_off, ok, 2, L, 8)
    assert st == 0 and not untouched
    # tree offsets that go backwards for the second tree: named, nothing written
    st, bt, bp, untouched = call_raw(ranks, path_off, np.array([0, 3, 2], np.int64), 2, L, 8)
    assert st == 1 and bt == 1 and bp == -1 and untouched
    # tree_off[0] != 0
    st, _, _, untouched = call_raw(ranks, path_off, np.array([1, 3, 4], np.int64), 2, L, 8)
    assert st == 1 and untouched
    # a path offset that goes backwards (in the second tree): nothing written
    bad_off = np.array([0, 1, 3, 2, 5], np.int64)
    st, _, _, untouched = call_raw(ranks, bad_off, ok, 2, L, 8)
    assert st == 1 and untouched
    # a prefix length out of range in the last tree: named, nothing written
    st, bt, _, untouched = call_raw(ranks, path_off, ok, 2, np.array([0, -5], np.int32), 8)
    assert st == 1 and bt == 1 and untouched
    # N outside 1..64
    assert call_raw(ranks, path_off, ok, 2, L, 0)[0] == 1
    assert call_raw(ranks, path_off, ok, 2, L, 65)[0] == 5
    # B == 0 is a no-op
    st, _, _, untouched = call_raw(ranks, path_off, np.array([0], np.int64), 0, L, 8)
    assert st == 0 and untouched


def test_relabelled_duplicates_and_order_within_each_tree():
    rng = np.random.Generator(np.random.PCG64(9))
    base = list(workloads.TEN_NODE_PATHS)
    trees = []
    for _ in range(6):
        t = base + [base[int(i)] for i in rng.integers(0, len(base), 3)]
        rng.shuffle(t)
        trees.append(t)
    L = rng.integers(0, 100, 6).astype(np.int32)
    got = tv.tree_meta_build_batch(PackedTrees(trees), L, 12)
    check_rows(trees, L, 12, got)


def test_prepared_build_repeats_into_the_same_arrays():
    # pointers resolved once; the prefix lengths and outputs keep their storage, and a
    # second call after the lengths change in place rebuilds the position ids
    rng = np.random.Generator(np.random.PCG64(73))
    trees = [workloads.random_tree(rng, n, 8)[0] for n in (33, 5, 20)]
    B, N = len(trees), 40
    L = np.array([100, 0, 4096], np.int32)
    out = {k: np.zeros((B, N), dt) for k, dt in (("parent", np.int32), ("depth", np.int32),
                                                  ("bitmask", np.uint64), ("pos", np.int32))}
    Lp = L.copy()   # the caller's int32 lengths are used in place, not copied
    build = tv.prepare_tree_meta_build_batch(PackedTrees(trees), Lp, N, out["parent"],
                                             out["depth"], out["bitmask"], out["pos"])
    for shift in (0, 7):
        Lp[:] = L + shift
        build()
        got = dict(out, num_nodes=build.num_nodes)
        check_rows(trees, L + shift, N, got)


def test_prepared_build_checks_its_outputs_and_reports_failures():
    trees = [list(workloads.TEN_NODE_PATHS), [(0,), (1, 0)]]
    good = np.zeros((2, 16), np.int32)
    with pytest.raises(ValueError):
        tv.prepare_tree_meta_build_batch(PackedTrees(trees), np.zeros(2, np.int32), 16,
                                         good, good.copy(), np.zeros((2, 16), np.int64),
                                         good.copy())
    build = tv.prepare_tree_meta_build_batch(PackedTrees(trees), np.zeros(2, np.int32), 16,
                                             good, good.copy(), np.zeros((2, 16), np.uint64),
                                             good.copy())
    with pytest.raises(TreeVerifyError) as e:
        build()
    assert e.value.name == "TV_ERR_MISSING_PARENT" and e.value.bad_tree == 1
