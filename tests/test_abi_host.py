"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, the
host builder matches the oracle bit-exactly, and every host-side argument check returns
its documented status without touching a device."""
import ctypes
import itertools
import os
import re
import subprocess

import numpy as np
import pytest

import tree_attention_draft_amd as tv
from oracle import meta
from tree_attention_draft_amd import workloads
from tree_attention_draft_amd._binding import TvAttnArgs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tree_verify.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = tv.lib()
    declared = declared_functions()
    assert set(declared) == set(tv.EXPORTS), declared
    nm = subprocess.run(["nm", "-D", "--defined-only", tv.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in nm.splitlines() if ln.strip()}
    for name in declared:
        assert name in exported, name
        assert getattr(L, name) is not None


def test_abi_struct_and_version():
    L = tv.lib()
    assert L.tv_abi_version() == 5
    assert L.tv_attn_args_sizeof() == ctypes.sizeof(TvAttnArgs)
    for code in range(8):
        assert L.tv_status_string(code).decode().startswith("TV_")


def test_pinned_device_address_rejects_null():
    # the argument checks come before any runtime call, so they hold without a device
    L = tv.lib()
    dev = ctypes.c_void_p(1)
    assert L.tv_pinned_device_address(None, ctypes.byref(dev)) == 1  # TV_ERR_INVALID_ARG
    x = ctypes.c_int32(0)
    assert L.tv_pinned_device_address(ctypes.byref(x), None) == 1
    assert "null" in L.tv_last_error().decode()


# --------------------------------------------------------------- host builder ----
def rank_paths_from_parent(parent):
    """Rank paths of a parent array: a child's rank is its order among its siblings."""
    paths = [()]
    seen = {}
    for i in range(1, len(parent)):
        p = parent[i]
        r = seen.get(p, 0)
        seen[p] = r + 1
        paths.append(paths[p] + (r,))
    return paths[1:]


def assert_same(paths, L):
    ref = meta.build_from_paths(paths, L)
    got = tv.tree_meta_build(paths, L)
    assert got["parent"].tolist() == ref["parent"]
    assert got["depth"].tolist() == ref["depth"]
    assert got["pos"].tolist() == ref["pos"]
    assert [int(x) for x in got["bitmask"]] == ref["bitmask"]


def test_builder_worked_example_chain_empty():
    assert_same(list(workloads.TEN_NODE_PATHS), 16)
    assert_same(workloads.chain_paths(5), 2048)
    assert_same([], 7)
    got = tv.tree_meta_build([], 7)
    assert got["parent"].tolist() == [-1] and got["bitmask"].tolist() == [1]


def test_builder_all_trees_up_to_6_nodes():
    for n in range(1, 7):
        for choice in itertools.product(*[range(i) for i in range(1, n)]):
            parent = [-1] + list(choice)
            assert_same(rank_paths_from_parent(parent), 3)


def test_builder_random_workload_trees_and_shuffles():
    rng = np.random.Generator(np.random.PCG64(21))
    for name in ("ragged64_n33", "wide32_n64", "long_paged_n33"):
        spec = workloads.WORKLOADS[name]
        trees, _ = workloads.trees_for(spec)
        for paths in trees:
            assert_same(paths, 100)
        # shuffled input with duplicates gives the same tree
        p = list(trees[0])
        shuffled = p + [p[i] for i in rng.integers(0, len(p), 5)]
        rng.shuffle(shuffled)
        ref = tv.tree_meta_build(p, 0)
        got = tv.tree_meta_build(shuffled, 0)
        for k in ref:
            assert np.array_equal(ref[k], got[k])


@pytest.mark.parametrize("scale,depth", [(1, 8), (127, 8), (128, 8), (1000, 10), (2 ** 30, 3)])
def test_builder_large_ranks_and_deep_paths(scale, depth):
    # the builder packs paths into 64-bit keys when ranks x length fit 56 bits (scale 1)
    # and compares them rank by rank otherwise (the larger scales); both agree with the
    # oracle, duplicates and shuffled input included
    rng = np.random.Generator(np.random.PCG64(scale + depth))
    for n in (5, 33, 64):
        parent, dep = [-1], [0]
        for i in range(1, n):
            choices = [j for j in range(i) if dep[j] < depth]
            parent.append(int(rng.choice(choices)))
            dep.append(dep[parent[-1]] + 1)
        paths = rank_paths_from_parent(parent)
        paths = [tuple(min(r * scale + (scale - 1 if r else 0), 2 ** 31 - 1) for r in p)
                 for p in paths]
        shuffled = list(paths) + [paths[i] for i in rng.integers(0, len(paths), 3)]
        rng.shuffle(shuffled)
        assert_same(shuffled, 5)
    bad = [(0,), (scale, 0), (0, scale)]       # (scale, 0) has no parent (scale,)
    with pytest.raises(meta.TreeError) as ref:
        meta.build_from_paths(bad, 0)
    with pytest.raises(tv.TreeVerifyError) as got:
        tv.tree_meta_build(bad, 0)
    assert got.value.bad_path == ref.value.index


@pytest.mark.parametrize("paths", [[(0, 0)], [(1,), (0, 1)], [(0,), (2, 0), (0, 0)],
                                   [(0,), (0, 0, 0)], [(3,), (0,), (0, 5, 1), (0, 4)]])
def test_builder_missing_parent_matches_oracle_index(paths):
    with pytest.raises(meta.TreeError) as ref:
        meta.build_from_paths(paths, 0)
    with pytest.raises(tv.TreeVerifyError) as got:
        tv.tree_meta_build(paths, 0)
    assert got.value.name == "TV_ERR_MISSING_PARENT"
    assert got.value.bad_path == ref.value.index


@pytest.mark.parametrize("paths,bad", [([(0,), ()], 1), ([(0,), (0, -1)], 1)])
def test_builder_invalid_paths(paths, bad):
    with pytest.raises(tv.TreeVerifyError) as e:
        tv.tree_meta_build(paths, 0)
    assert e.value.name == "TV_ERR_INVALID_PATH" and e.value.bad_path == bad


def test_builder_capacity():
    paths = [(i,) for i in range(63)]
    assert len(tv.tree_meta_build(paths, 0)["parent"]) == 64
    with pytest.raises(tv.TreeVerifyError) as e:
        tv.tree_meta_build(paths + [(63,)], 0, max_nodes=64)
    assert e.value.name == "TV_ERR_CAPACITY"
    with pytest.raises(tv.TreeVerifyError) as e:
        tv.tree_meta_build(paths[:5], 0, max_nodes=5)
    assert e.value.name == "TV_ERR_CAPACITY"
    with pytest.raises(tv.TreeVerifyError) as e:
        tv.tree_meta_build(paths + [(63,)], 0, max_nodes=100)
    assert e.value.name == "TV_ERR_CAPACITY"


def test_builder_bad_arguments():
    L = tv.lib()
    buf = np.zeros(8, np.int64)
    out = np.zeros(64, np.int64)
    n = ctypes.c_int32()
    # negative num_paths, null outputs, bad offsets, negative prefix
    assert L.tree_meta_build(None, buf.ctypes.data, -1, 0, 64, out.ctypes.data,
                             out.ctypes.data, out.ctypes.data, out.ctypes.data,
                             ctypes.byref(n), None) == 1
    assert L.tree_meta_build(None, buf.ctypes.data, 0, 0, 64, None, None, None, None,
                             None, None) == 1
    offs = np.array([0, 2, 1], np.int64)
    ranks = np.zeros(4, np.int32)
    assert L.tree_meta_build(ranks.ctypes.data, offs.ctypes.data, 2, 0, 64, out.ctypes.data,
                             out.ctypes.data, out.ctypes.data, out.ctypes.data,
                             ctypes.byref(n), None) == 1
    offs = np.array([0, 1], np.int64)
    assert L.tree_meta_build(ranks.ctypes.data, offs.ctypes.data, 1, -5, 64,
                             out.ctypes.data, out.ctypes.data, out.ctypes.data,
                             out.ctypes.data, ctypes.byref(n), None) == 1


# --------------------------------------------------------------- attn validation -
def base_args(**kw):
    a = TvAttnArgs()
    a.dtype, a.B, a.N, a.Hq, a.Hkv, a.D = 0, 2, 10, 32, 8, 128
    fake = 1 << 20  # aligned, never dereferenced: validation fails before any launch
    a.q = a.k = a.v = a.out = fake
    a.parent = a.prefix_len = fake
    a.q_sb, a.q_sn, a.q_sh = 10 * 32 * 128, 32 * 128, 128
    a.kv_sb, a.kv_st, a.kv_sh = 100 * 8 * 128, 8 * 128, 128
    a.o_sb, a.o_sn, a.o_sh = a.q_sb, a.q_sn, a.q_sh
    a.parent_sb = 10
    a.max_prefix_len = 64
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 1), (dict(N=65), 5), (dict(Hq=30), 1), (dict(Hkv=0), 1),
    (dict(D=96), 5), (dict(dtype=7), 1), (dict(B=-1), 1), (dict(q=None), 1),
    (dict(parent=None), 1), (dict(prefix_len=None), 1), (dict(out=None), 1),
    (dict(q_sn=100), 1), (dict(kv_st=-8), 1), (dict(k=(1 << 20) + 8), 1),
    (dict(parent_sb=3), 1), (dict(max_prefix_len=-1), 1), (dict(sm_scale=-1.0), 1),
    (dict(sm_scale=float("inf")), 1), (dict(num_splits=-2), 1), (dict(path=9), 1),
    (dict(path=2, dtype=1), 5), (dict(kv_layout=1), 1),
    (dict(kv_layout=1, page_table=1 << 20, page_size=16, pages_per_seq=4), 1),
    (dict(kv_layout=3), 1), (dict(rope_theta=-1.0), 1), (dict(rope_theta=float("nan")), 1),
    (dict(rope_theta=float("inf")), 1),
])
def test_attn_argument_checks(kw, status):
    a = base_args(**kw)
    L = tv.lib()
    assert L.tree_verify_attn(ctypes.byref(a), None) == status
    assert L.tv_last_error().decode() != ""
    pointer_only = any(k in ("q", "k", "parent", "prefix_len", "out") for k in kw)
    if not pointer_only:
        assert L.tree_verify_attn_workspace_size(ctypes.byref(a)) == 0


def test_workspace_size_ignores_pointers():
    a = base_args(B=1, max_prefix_len=32768, num_splits=8, q=None, k=None, v=None,
                  out=None, parent=None, prefix_len=None)
    assert tv.lib().tree_verify_attn_workspace_size(ctypes.byref(a)) == 8 * 8 * 40 * 129 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 1), (dict(N=65), 5), (dict(D=96), 5), (dict(q=None), 1), (dict(B=-1), 1)])
def test_static_entry_point_shares_the_argument_checks(kw, status):
    assert tv.lib().tree_verify_attn_static(ctypes.byref(base_args(**kw)), None) == status


def test_static_entry_point_rejects_plans_beyond_its_array():
    # B=8, L=32768, 64 splits (57 after rounding): 8*8*57*40*129*4 bytes > 64 MiB; refused
    # before any device call (the workspace argument is ignored: a large one does not help)
    a = base_args(B=8, max_prefix_len=32768, num_splits=64, workspace=1 << 20,
                  workspace_bytes=1 << 40)
    assert tv.lib().tree_verify_attn_workspace_size(ctypes.byref(a)) > tv.STATIC_SCRATCH_BYTES
    assert tv.lib().tree_verify_attn_static(ctypes.byref(a), None) == 6
    assert "static scratch" in tv.lib().tv_last_error().decode()


def test_attn_empty_batch_is_noop():
    a = base_args(B=0, q=None, k=None, v=None, out=None, parent=None, prefix_len=None)
    assert tv.lib().tree_verify_attn(ctypes.byref(a), None) == 0


def test_workspace_missing_is_rejected_before_launch():
    # B=1, long prefix: the plan splits keys, so a workspace is required
    a = base_args(B=1, max_prefix_len=32768, num_splits=8)
    need = tv.lib().tree_verify_attn_workspace_size(ctypes.byref(a))
    R = 10 * 4
    assert need == 1 * 8 * 8 * R * (128 + 1) * 4
    assert tv.lib().tree_verify_attn(ctypes.byref(a), None) == 6
    a.workspace, a.workspace_bytes = 1 << 20, need - 4
    assert tv.lib().tree_verify_attn(ctypes.byref(a), None) == 6


def ragged_args(lengths, hint):
    """B=len(lengths) requests, N=33, 32q/8kv, D=128, bf16, bound = max length; the host
    copy of the lengths is attached only when `hint`."""
    B = len(lengths)
    lens = np.asarray(lengths, np.int32)
    a = base_args(B=B, N=33, max_prefix_len=int(lens.max()), parent_sb=33,
                  q_sb=33 * 32 * 128, q_sn=32 * 128, o_sb=33 * 32 * 128, o_sn=32 * 128)
    if hint:
        a._hint = lens
        a.prefix_len_host = lens.ctypes.data
    return a


def test_split_plan_from_host_lengths():
    # (the automatic plan assumes 2 workgroups per compute unit; no GPU here: 256 units)
    rng = np.random.Generator(np.random.PCG64(7))
    ragged = rng.integers(512, 8193, size=64)
    ragged[0] = 8192                        # the bound: 129 key tiles of 64
    L = tv.lib()
    R, D, Hkv = 33 * 4, 128, 8
    # without the lengths the plan sees 64 requests of 8192 keys: they fill the slots
    assert L.tree_verify_attn_workspace_size(ctypes.byref(ragged_args(ragged, False))) == 0
    # with them it sizes chunks to the average work per workgroup slot (74 key tiles) and
    # splits the long requests in two
    work = sum((int(x) + 33 + 63) // 64 for x in ragged) * Hkv
    chunk = -(-work // 512)
    S = -(-129 // chunk)
    assert chunk == 74 and S == 2
    got = L.tree_verify_attn_workspace_size(ctypes.byref(ragged_args(ragged, True)))
    assert got == 64 * Hkv * S * R * (D + 1) * 4
    # equal lengths: the hint changes nothing
    same = np.full(64, 4096)
    for hint in (False, True):
        assert L.tree_verify_attn_workspace_size(ctypes.byref(ragged_args(same, hint))) == 0
    # a small batch splits with or without the lengths
    small = [2048] * 8
    a0 = L.tree_verify_attn_workspace_size(ctypes.byref(ragged_args(small, False)))
    a1 = L.tree_verify_attn_workspace_size(ctypes.byref(ragged_args(small, True)))
    assert a0 == a1 > 0


def test_single_split_needs_no_workspace():
    a = base_args(num_splits=1)
    assert tv.lib().tree_verify_attn_workspace_size(ctypes.byref(a)) == 0


def test_meta_from_parent_argument_checks():
    L = tv.lib()
    assert L.tree_meta_from_parent(1 << 20, 0, 4, 0, None, None, None, None, None) == 1
    assert L.tree_meta_from_parent(1 << 20, 0, 4, 65, None, None, None, None, None) == 5
    assert L.tree_meta_from_parent(1 << 20, 5, 4, 10, None, None, None, None, None) == 1
    assert L.tree_meta_from_parent(None, 0, 4, 10, None, None, None, None, None) == 1
    assert L.tree_meta_from_parent(None, 0, 0, 10, None, None, None, None, None) == 0


# ------------------------------------------------- acceptance / compaction checks ----
def base_accept_args(**kw):
    a = tv.TvAcceptArgs()
    a.dtype, a.B, a.N, a.V = 0, 2, 10, 1000
    fake = 1 << 20  # never dereferenced: every case below fails validation first
    a.logits = a.tokens = a.parent = fake
    a.target = a.accepted = a.emitted = a.num_accepted = fake
    a.workspace, a.workspace_bytes = fake, 2 * 10 * 8
    a.lg_sb, a.lg_sn = 10 * 1000, 1000
    a.tokens_sb = a.parent_sb = 10
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_accept_rejects_trees_above_64_nodes_as_unsupported():
    L = tv.lib()
    assert L.tree_accept_greedy(ctypes.byref(base_accept_args(N=65)), None) == 5


@pytest.mark.parametrize("kw", [
    dict(N=0), dict(V=0), dict(B=-1), dict(dtype=5), dict(logits=None),
    dict(tokens=None), dict(parent=None), dict(target=None), dict(accepted=None),
    dict(emitted=None), dict(num_accepted=None), dict(lg_sn=999), dict(lg_sb=5000),
    dict(tokens_sb=3), dict(parent_sb=9), dict(logits=(1 << 20) + 1),
])
def test_accept_argument_checks(kw):
    L = tv.lib()
    assert L.tree_accept_greedy(ctypes.byref(base_accept_args(**kw)), None) == 1
    assert L.tv_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(workspace=None), 6), (dict(workspace_bytes=2 * 10 * 8 - 1), 6),
    (dict(workspace=(1 << 20) + 4), 1), (dict(B=7000, lg_sb=10 * 1000), 5),
])
def test_accept_workspace_checks(kw, status):
    a = base_accept_args(**kw)
    L = tv.lib()
    assert L.tree_accept_greedy(ctypes.byref(a), None) == status
    assert L.tree_accept_greedy_workspace_size(ctypes.byref(base_accept_args())) == 2 * 10 * 8
    # one key per 8192-entry slice of every row
    big = base_accept_args(V=128256, lg_sn=128256, lg_sb=10 * 128256)
    assert L.tree_accept_greedy_workspace_size(ctypes.byref(big)) == 2 * 10 * 16 * 8
    big.workspace_bytes = 2 * 10 * 16 * 8 - 1
    assert L.tree_accept_greedy(ctypes.byref(big), None) == 6


def test_accept_empty_batch_is_noop():
    a = base_accept_args(B=0, logits=None, tokens=None, parent=None, target=None)
    assert tv.lib().tree_accept_greedy(ctypes.byref(a), None) == 0


def base_sample_args(**kw):
    a = tv.TvSampleArgs()
    a.B, a.N, a.V = 2, 10, 1000
    fake = 1 << 20  # never dereferenced: every case below fails validation first
    a.p = a.q = a.tokens = a.parent = a.uniform = fake
    a.accepted = a.emitted = a.num_accepted = fake
    a.p_sb = a.q_sb = 10 * 1000
    a.p_sn = a.q_sn = 1000
    a.tokens_sb = a.parent_sb = a.uniform_sb = 10
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 1), (dict(V=0), 1), (dict(B=-1), 1), (dict(N=65), 5), (dict(B=70000), 5),
    (dict(p=None), 1), (dict(q=None), 1), (dict(tokens=None), 1), (dict(parent=None), 1),
    (dict(uniform=None), 1), (dict(accepted=None), 1), (dict(emitted=None), 1),
    (dict(num_accepted=None), 1), (dict(p_sn=999), 1), (dict(q_sb=5000), 1),
    (dict(p_sb=-1), 1), (dict(tokens_sb=3), 1), (dict(parent_sb=9), 1),
    (dict(uniform_sb=9), 1), (dict(p=(1 << 20) + 2), 1), (dict(uniform=(1 << 20) + 4), 1),
])
def test_stochastic_accept_argument_checks(kw, status):
    L = tv.lib()
    assert L.tree_accept_stochastic(ctypes.byref(base_sample_args(**kw)), None) == status
    assert L.tv_last_error().decode() != ""


def test_stochastic_accept_empty_batch_is_noop():
    a = base_sample_args(B=0, p=None, q=None, tokens=None, parent=None, uniform=None)
    assert tv.lib().tree_accept_stochastic(ctypes.byref(a), None) == 0


def base_compact_args(**kw):
    a = tv.TvCompactArgs()
    a.dtype, a.B, a.N, a.Hkv, a.D = 0, 2, 10, 8, 128
    fake = 1 << 20
    a.k = a.v = a.prefix_len = a.parent = a.accepted = a.num_accepted = fake
    a.kv_sb, a.kv_st, a.kv_sh = 100 * 8 * 128, 8 * 128, 128
    a.parent_sb = 10
    a.max_prefix_len = 64
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 1), (dict(N=65), 5), (dict(Hkv=0), 1), (dict(D=96), 5), (dict(B=-1), 1),
    (dict(dtype=4), 1), (dict(kv_layout=2), 1), (dict(k=None), 1), (dict(v=None), 1),
    (dict(prefix_len=None), 1), (dict(parent=None), 1), (dict(accepted=None), 1),
    (dict(num_accepted=None), 1), (dict(kv_st=-8), 1), (dict(kv_sh=4), 1),
    (dict(k=(1 << 20) + 8), 1), (dict(parent_sb=5), 1), (dict(max_prefix_len=-1), 1),
    (dict(kv_layout=1), 1),
    (dict(kv_layout=1, page_table=1 << 20, page_size=16, pages_per_seq=4), 1),
    (dict(rope_theta=-2.0), 1), (dict(rope_theta=float("nan")), 1),
])
def test_compact_argument_checks(kw, status):
    L = tv.lib()
    assert L.tree_kv_compact(ctypes.byref(base_compact_args(**kw)), None) == status
    assert L.tv_last_error().decode() != ""


def test_compact_empty_batch_is_noop():
    a = base_compact_args(B=0, k=None, v=None, prefix_len=None)
    assert tv.lib().tree_kv_compact(ctypes.byref(a), None) == 0


def test_after_pass_struct_sizes():
    L = tv.lib()
    assert L.tv_accept_args_sizeof() == ctypes.sizeof(tv.TvAcceptArgs)
    assert L.tv_sample_args_sizeof() == ctypes.sizeof(tv.TvSampleArgs)
    assert L.tv_compact_args_sizeof() == ctypes.sizeof(tv.TvCompactArgs)
