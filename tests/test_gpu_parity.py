"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Tolerances: max-abs 2e-2 on outputs and LSE for bf16 inputs (fp32 accumulation), 1e-5
for fp32 inputs; tree metadata bit-exact.  Small cases are checked in full; the full-size
workloads in the launch configuration the benchmark times are checked on sampled
requests (every node and head of each sampled request).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
import tree_attention_draft_amd as tv  # noqa: E402
from oracle import meta as ometa  # noqa: E402
from tree_attention_draft_amd import workloads  # noqa: E402

from gpu_cases import Case, StreamedPagedCase, say  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TEN = list(workloads.TEN_NODE_PATHS)


def random_trees(seed, B, n, cap):
    rng = np.random.Generator(np.random.PCG64(seed))
    paths, creation = [], []
    for _ in range(B):
        p, c = workloads.random_tree(rng, n, cap)
        paths.append(p)
        creation.append(c)
    return paths, creation


# ------------------------------------------------------------------ metadata ----------
def test_meta_from_parent_bit_exact():
    cases = []
    paths, creation = random_trees(2003, 64, 33, 8)
    cases.append(("random33", [ometa.build_from_paths(p, 0)["parent"] for p in paths]))
    cases.append(("creation_order33", creation))
    paths64, _ = random_trees(2004, 32, 64, 10)
    cases.append(("random64", [ometa.build_from_paths(p, 0)["parent"] for p in paths64]))
    cases.append(("tree10", [ometa.build_from_paths(TEN, 0)["parent"]] * 3))
    cases.append(("chain5", [[-1, 0, 1, 2, 3]] * 2))
    cases.append(("empty", [[-1]] * 5))
    for name, parents in cases:
        say("meta_from_parent", name)
        P = torch.tensor(np.array(parents, np.int32)).cuda()
        L = torch.arange(P.shape[0], dtype=torch.int32).cuda() * 100 + 7
        depth, bitmask, pos = tv.tree_meta_from_parent(P, L)
        depth, bitmask, pos = depth.cpu().numpy(), bitmask.cpu().numpy(), pos.cpu().numpy()
        for b, par in enumerate(parents):
            ref = ometa.meta_from_parent(par, 100 * b + 7)
            assert depth[b].tolist() == ref["depth"]
            assert pos[b].tolist() == ref["pos"]
            assert [int(x) & (2 ** 64 - 1) for x in bitmask[b]] == ref["bitmask"]


def test_meta_from_parent_shared_tree_and_invalid_nodes():
    par = ometa.build_from_paths(TEN, 0)["parent"]
    P = torch.tensor(par, dtype=torch.int32).cuda()
    L = torch.tensor([5, 9, 11], dtype=torch.int32).cuda()
    depth, bitmask, pos = tv.tree_meta_from_parent(P, L)   # one tree, 3 requests
    for b, Lb in enumerate([5, 9, 11]):
        ref = ometa.meta_from_parent(par, Lb)
        assert pos[b].cpu().tolist() == ref["pos"]
        assert [int(x) for x in bitmask[b].cpu()] == ref["bitmask"]
    # broken conventions are flagged node by node, never read out of bounds
    bad = torch.tensor([[-1, 0, 2, 1, 7], [3, 0, 1, 2, 3], [-1, 0, 1, -1, 3]],
                       dtype=torch.int32).cuda()
    depth, bitmask, pos = tv.tree_meta_from_parent(bad)
    d = depth.cpu().tolist()
    assert d[0] == [0, 1, -1, 2, -1]
    assert d[1] == [-1, -1, -1, -1, -1]
    assert d[2] == [0, 1, 2, -1, -1]
    assert int(bitmask[0, 1]) == 0b11 and int(bitmask[0, 2]) == 0


def _meta_ref(parents, L):
    return [ometa.meta_from_parent(list(par), int(Lb)) for par, Lb in zip(parents, L)]


def _meta_outputs(B, N):
    return (torch.full((B, N), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, N), -7, dtype=torch.int64, device="cuda"),
            torch.full((B, N), -7, dtype=torch.int32, device="cuda"))


def _assert_meta(meta, refs):
    depth, bitmask, pos = (t.cpu().numpy() for t in meta)
    for b, ref in enumerate(refs):
        assert depth[b].tolist() == ref["depth"], b
        assert pos[b].tolist() == ref["pos"], b
        assert [int(x) & (2 ** 64 - 1) for x in bitmask[b]] == ref["bitmask"], b


@pytest.mark.parametrize("shape", ["mfma_splits", "mfma_longest_first", "mfma_node_chunks",
                                   "mfma_rope", "valu_f32"])
def test_pass_exports_tree_metadata(shape):
    # the pass expands the parent arrays in its prologue; written out, that expansion
    # equals the oracle's metadata bit for bit and leaves out/lse bit-identical
    if shape == "mfma_splits":
        paths, _ = random_trees(2600, 5, 33, 8)
        c = Case("meta_export_splits", [100, 900, 0, 513, 64], trees=paths, seed=2601)
        kw = dict(num_splits=3)
    elif shape == "mfma_longest_first":
        rng = np.random.Generator(np.random.PCG64(2602))
        L = rng.integers(1, 2000, size=12).astype(np.int32)
        paths, _ = random_trees(2603, 12, 17, 6)
        c = Case("meta_export_lpt", L, trees=paths, seed=2604)
        kw = dict(prefix_len_host=L)
    elif shape == "mfma_node_chunks":
        paths, _ = random_trees(2605, 3, 64, 10)
        c = Case("meta_export_n64", [300, 40, 1000], trees=paths, Hq=64, Hkv=8, seed=2606)
        kw = {}
    elif shape == "mfma_rope":
        paths, _ = random_trees(2609, 4, 33, 8)
        c = Case("meta_export_rope", [700, 31, 64, 1500], trees=paths, seed=2610)
        kw = dict(rope_theta=10000.0, num_splits=2)
    else:
        c = Case("meta_export_f32", [16, 3, 40], trees=TEN, Hq=1, Hkv=1, D=64, dtype="f32",
                 seed=2607)
        kw = dict(num_splits=2)
    out0, lse0 = c.run(**kw)
    meta = _meta_outputs(c.B, c.N)
    out1, lse1 = c.run(meta=meta, **kw)
    _assert_meta(meta, _meta_ref(c.parent_oracle, c.L))
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)
    c.check(out1, lse1)


def test_pass_exports_flag_invalid_nodes():
    # broken parent conventions: the export flags them node by node exactly as the
    # standalone kernel does (the attention results of such trees are unspecified)
    bad = [[-1, 0, 2, 1, 7], [-1, 0, 1, -1, 3], [-1, 0, 0, 1, 2]]
    c = Case("meta_export_invalid", [20, 50, 8], parents=bad, Hq=4, Hkv=1, D=64, seed=2608)
    meta = _meta_outputs(c.B, c.N)
    c.run(meta=meta)
    P = torch.tensor(np.array(bad, np.int32)).cuda()
    ref = tv.tree_meta_from_parent(P, c.device()["prefix_len"])
    for got, want in zip(meta, ref):
        assert torch.equal(got, want)
    assert meta[0].cpu().tolist()[0] == [0, 1, -1, 2, -1]


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 32, 8, 128), ("f32", 2, 1, 64)])
def test_pinned_host_parent_read_in_place(dtype, Hq, Hkv, D):
    # the parent arrays may stay in pinned host memory: the pass reads them in place
    paths, _ = random_trees(2610, 4, 33, 8)
    c = Case(f"pinned_parent_{dtype}", [300, 1000, 77, 2048], trees=paths, Hq=Hq, Hkv=Hkv,
             D=D, dtype=dtype, seed=2611)
    out_d, lse_d = c.run(num_splits=2)
    host_parent = torch.tensor(np.array(c.parent_gpu, np.int32)).pin_memory()
    meta = _meta_outputs(c.B, c.N)
    out_h, lse_h = c.run(parent=host_parent, num_splits=2, meta=meta)
    assert np.array_equal(out_d, out_h) and np.array_equal(lse_d, lse_h)
    _assert_meta(meta, _meta_ref(c.parent_oracle, c.L))
    c.check(out_h, lse_h)
    with pytest.raises(ValueError):
        c.run(parent=torch.tensor(np.array(c.parent_gpu, np.int32)))  # pageable host memory


# ------------------------------------------------------------------ worked example ----
@pytest.mark.parametrize("tree", ["tree10", "empty", "chain5"])
@pytest.mark.parametrize("splits", [0, 1, 2])
def test_single_request_fp32(tree, splits):
    trees = {"tree10": TEN, "empty": [], "chain5": workloads.chain_paths(5)}[tree]
    c = Case(f"{tree}_f32", [16], trees=trees, Hq=1, Hkv=1, D=64, dtype="f32", seed=1001)
    out, lse = c.run(num_splits=splits)
    c.check(out, lse)


@pytest.mark.parametrize("tree", ["tree10", "chain5"])
def test_llama8b_shape_full(tree):
    trees = TEN if tree == "tree10" else workloads.chain_paths(5)
    c = Case(f"llama8b_{tree}", [2048] * 8, trees=trees, seed=1002)
    out, lse = c.run()
    c.check(out, lse)


# ------------------------------------------------------------------ shapes & paths ----
@pytest.mark.parametrize("N", [1, 2, 5, 10, 16, 17, 33, 49, 50, 63, 64])
def test_node_count_sweep(N):
    paths, _ = random_trees(500 + N, 2, N, 8)
    c = Case(f"nodes{N}", [300, 77], trees=paths, seed=1100 + N)
    out, lse = c.run()
    c.check(out, lse)


# Small grids (at most one workgroup per compute unit) run the two-team build: every
# four-wave shape -- one, two or three 16-node tiles per wave, with and without the shared
# remainder tile, and trees of one node and of exactly one full tile -- over key ranges of
# 1 to 9 tiles, so a window is often half empty or one team has no tile at all, and one of
# 32 tiles (eight windows), with and without forced splits (several 32-key tiles per
# split, and splits of one chunk).
@pytest.mark.parametrize("N", [1, 5, 10, 16, 17, 32, 33, 48])
@pytest.mark.parametrize("splits", [0, 3])
def test_team_shapes(N, splits):
    paths, _ = random_trees(900 + N, 5, N, 8)
    c = Case(f"teams_n{N}_s{splits}", [0, 20, 97, 240, 1000], trees=paths, seed=1500 + N)
    out, lse = c.run(num_splits=splits)
    c.check(out, lse)


@pytest.mark.parametrize("hq,hkv", [(64, 4), (16, 8), (8, 1)])
def test_group_sizes_n33(hq, hkv):
    # g = 16 (two head chunks of 8 waves), g = 2, g = 8 with one kv head
    paths, _ = random_trees(800 + hq, 2, 33, 8)
    c = Case(f"groups{hq}_{hkv}", [515, 64], trees=paths, Hq=hq, Hkv=hkv, seed=1400 + hq)
    out, lse = c.run()
    c.check(out, lse)


@pytest.mark.parametrize("dtype,path", [("bf16", "mfma"), ("bf16", "valu"), ("f32", "valu")])
@pytest.mark.parametrize("scale", [0.02, 0.35])
def test_explicit_softmax_scale(dtype, path, scale):
    # a small scale (flat weights) and a large one (peaked weights, frequent rebasing)
    paths, _ = random_trees(900, 2, 33, 8)
    c = Case(f"scale{scale}_{dtype}_{path}", [700, 96], trees=paths, dtype=dtype,
             seed=1500 + int(scale * 100))
    out, lse = c.run(sm_scale=scale, path=path)
    c.check(out, lse)


@pytest.mark.parametrize("N", [64])
@pytest.mark.parametrize("hq,hkv", [(64, 8), (16, 8)])
def test_node_chunks(N, hq, hkv):
    # 64 nodes = four 16-node tiles per head: split over two workgroups per kv head
    paths, _ = random_trees(700 + hq, 3, N, 10)
    c = Case(f"nodechunks{hq}_{hkv}", [1000, 33, 0], trees=paths, Hq=hq, Hkv=hkv,
             seed=1300 + hq)
    for splits in (0, 3):
        out, lse = c.run(num_splits=splits)
        c.check(out, lse)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (16, 2)])
def test_head_shapes_and_forced_paths(D, hq, hkv):
    paths, _ = random_trees(600, 3, 12, 5)
    c = Case(f"heads{hq}_{hkv}_D{D}", [130, 64, 1], trees=paths, Hq=hq, Hkv=hkv, D=D,
             seed=1200 + D + hq)
    results = {}
    for path in ("auto", "valu", "mfma"):
        out, lse = c.run(path=path)
        c.check(out, lse)
        results[path] = out
    assert np.abs(results["valu"] - results["mfma"]).max() <= 2e-2


# Requested split counts 1, 2, 7, 9, 20 and 1000 give grids of 1, 2, 7, 8, 16 and 64
# splits over the longest request (64 chunks of 64 keys): the merge then spreads each
# output's partials over 1, 2, 4 or 8 thread groups; the shorter requests have fewer
# partials than the grid (and the 33-key one a single chunk, written directly).
@pytest.mark.parametrize("splits", [1, 2, 7, 9, 20, 1000])
def test_split_invariance(splits):
    paths, _ = random_trees(700, 3, 33, 8)
    c = Case("splits", [4000, 999, 33], trees=paths, seed=1300)
    out, lse = c.run(num_splits=splits)
    c.check(out, lse)


@pytest.mark.parametrize("splits", [3, 1000])
def test_split_invariance_d64(splits):
    # D = 64: two output rows per merge workgroup at eight thread groups per output
    paths, _ = random_trees(710, 3, 17, 8)
    c = Case("splits_d64", [2500, 130, 700], trees=paths, Hq=16, Hkv=4, D=64, seed=1310)
    out, lse = c.run(num_splits=splits)
    c.check(out, lse)


@pytest.mark.parametrize("splits", [12, 1000])
def test_split_invariance_f32(splits):
    # the vector path (fp32) with 2 and 8 merge thread groups per output (64-key chunks:
    # 48 of them over the longest request)
    c = Case("splits_f32", [3000, 64, 777], trees=TEN, Hq=4, Hkv=2, D=64, dtype="f32",
             seed=1330)
    out, lse = c.run(num_splits=splits)
    c.check(out, lse)


def test_prepared_call_matches_the_plain_call():
    # arguments marshalled once, the call repeated with the same buffers: bit-identical to
    # the plain call, also after the inputs change in place between calls
    import torch
    paths, _ = random_trees(720, 3, 33, 8)
    c = Case("prepared", [900, 40, 3000], trees=paths, seed=1320)
    d = c.device()
    Lmax = int(c.L.max())
    out = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[:3], dtype=torch.float32, device="cuda")
    call = tv.prepare_tree_verify_attn(d["q"], d["k"], d["v"], d["parent"], d["prefix_len"],
                                       Lmax, out=out, lse=lse, num_splits=5)
    for scale in (1.0, 0.5):
        d["q"].mul_(scale)
        want_o, want_l = tv.tree_verify_attn(d["q"], d["k"], d["v"], d["parent"],
                                             d["prefix_len"], Lmax, num_splits=5)
        got_o, got_l = call()
        torch.cuda.synchronize()
        assert got_o is out and got_l is lse
        assert torch.equal(got_o, want_o) and torch.equal(got_l, want_l), scale
    d["q"].mul_(2.0)  # back to the inputs the oracle reads (scaling by 0.5 and 2 is exact)
    call()
    torch.cuda.synchronize()
    c.check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))


def test_prefix_edges_in_one_batch():
    Ls = [0, 1, 63, 64, 65, 127, 128, 129, 5]
    paths, _ = random_trees(800, len(Ls), 33, 8)
    c = Case("prefix_edges", Ls, trees=paths, seed=1400)
    for splits in (0, 1, 3):
        out, lse = c.run(num_splits=splits)
        c.check(out, lse)


def test_fp32_larger_rows_valu():
    paths, _ = random_trees(900, 2, 20, 6)
    c = Case("f32_rows", [200, 333], trees=paths, Hq=8, Hkv=2, D=128, dtype="f32",
             seed=1500)
    out, lse = c.run()
    c.check(out, lse)
    out, lse = c.run(num_splits=4)
    c.check(out, lse)


# ------------------------------------------------------------------ invariants --------
def test_non_ancestor_edits_leave_node_bit_identical():
    par = ometa.build_from_paths(TEN, 0)["parent"]
    c = Case("edit_nonancestor", [200, 200], parents=[par, par], seed=1600)
    base, base_lse = c.run()
    d = c.device()
    node = 9
    anc = {9, 6, 3, 1, 0}
    k2, v2 = d["k"].clone(), d["v"].clone()
    for j in range(len(par)):
        if j not in anc:
            k2[:, 200 + j] = torch.randn_like(k2[:, 200 + j].float()).to(k2.dtype) * 50
            v2[:, 200 + j] = torch.randn_like(v2[:, 200 + j].float()).to(v2.dtype) * 50
    out, lse = tv.tree_verify_attn(d["q"], k2, v2, d["parent"], d["prefix_len"], 200)
    out = out.float().cpu().numpy()
    assert np.array_equal(out[:, node], base[:, node])
    assert np.array_equal(lse.cpu().numpy()[:, node], base_lse[:, node])


def test_relabelling_permutes_outputs():
    paths, creation = random_trees(1000, 2, 33, 8)
    canon = [ometa.build_from_paths(p, 0) for p in paths]
    c1 = Case("canonical", [400, 250], trees=paths, seed=1700)
    out1, lse1 = c1.run()
    c1.check(out1, lse1)
    # same tokens stored in creation order: Q rows and tree K/V rows permuted
    c2 = Case("creation_order", [400, 250], parents=creation, seed=1700)
    for b in range(2):
        index = {p: i for i, p in enumerate(canon[b]["paths"])}
        perm = [index[p] for p in [()] + paths[b]]        # creation i -> canonical
        L = [400, 250][b]
        for key in ("k", "v"):
            c2.host[key][b, L:L + 33] = c1.host[key][b, L:L + 33][perm]
        c2.host["q"][b] = c1.host["q"][b][perm]
    out2, lse2 = c2.run()
    c2.check(out2, lse2)
    for b in range(2):
        index = {p: i for i, p in enumerate(canon[b]["paths"])}
        perm = [index[p] for p in [()] + paths[b]]
        assert np.abs(out2[b] - out1[b][perm]).max() <= 2e-2


def test_rising_scores_take_the_overflow_fallback():
    # Every query is the same +-1 vector u and prefix key t is u * t/64, so the scores grow
    # by about 0.14 log2 units per key at this scale: far past the 64-unit weight bound
    # several times per request, which the fast softmax step must catch and rebase.
    paths, _ = random_trees(1900, 2, 33, 8)
    c = Case("rising_scores", [1024, 700], trees=paths, seed=1900)
    rng = np.random.Generator(np.random.PCG64(1901))
    u = np.where(rng.random(128) < 0.5, -1.0, 1.0).astype(np.float32)
    c.host["q"][:] = workloads.f32_to_bf16_bits(np.broadcast_to(u, c.host["q"].shape).copy(),
                                                finite=True)
    for b, L in enumerate(c.L):
        ramp = (np.arange(L, dtype=np.float32) / 64.0)[:, None, None] * u
        c.host["k"][b, :L] = workloads.f32_to_bf16_bits(
            np.broadcast_to(ramp, (L, c.Hkv, 128)).copy(), finite=True)
    out, lse = c.run(sm_scale=0.05)
    c.check(out, lse)


def test_shared_tree_strided_tensors_and_no_lse():
    par = ometa.build_from_paths(TEN, 0)["parent"]
    c = Case("shared_strided", [300, 301, 302], parents=[par] * 3, seed=1800)
    d = c.device()
    big_q = torch.zeros((3, 10, 40, 128), dtype=torch.bfloat16, device="cuda")
    big_q[:, :, 4:36] = d["q"]
    q_view = big_q[:, :, 4:36]                      # non-contiguous head stride window
    out_big = torch.full((3, 12, 32, 136), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_view = out_big[:, 1:11, :, :128]
    shared = torch.tensor(par, dtype=torch.int32, device="cuda")
    tv.tree_verify_attn(q_view, d["k"], d["v"], shared, d["prefix_len"], 302, out=out_view)
    ref_out, ref_lse = c.run()
    got = out_view.float().cpu().numpy()
    assert np.array_equal(got, ref_out)
    assert torch.isnan(out_big[:, 0].float()).all() and torch.isnan(out_big[:, 11].float()).all()
    # lse may be omitted (NULL)
    a = tv.make_args(d["q"], d["k"], d["v"], d["parent"], d["prefix_len"], 302,
                     out=torch.empty_like(d["q"]), num_splits=1)
    import ctypes
    st = tv.lib().tree_verify_attn(ctypes.byref(a),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0


def test_empty_batch_noop():
    q = torch.empty((0, 5, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 10, 8, 128), dtype=torch.bfloat16, device="cuda")
    par = torch.empty((0, 5), dtype=torch.int32, device="cuda")
    pl = torch.empty((0,), dtype=torch.int32, device="cuda")
    out, lse = tv.tree_verify_attn(q, k, k, par, pl, 0)
    assert out.shape == (0, 5, 32, 128)


# ------------------------------------------------------------------ workloads ---------
def test_ragged_small_full():
    spec = workloads.WORKLOADS["ragged64_n33"]
    trees, _ = workloads.trees_for(spec)
    L = workloads.prefix_lengths(spec)[:6] // 4
    c = Case("ragged_small", L, trees=trees[:6], seed=1003)
    out, lse = c.run()
    c.check(out, lse)
    # with the host copy of the lengths: chunks sized to the total work, requests taken
    # longest first, short requests written directly, the rest merged
    out, lse = c.run(prefix_len_host=c.L)
    c.check(out, lse)


@pytest.mark.parametrize("B", [12, 64, 300])
def test_ragged_host_lengths(B):
    # lengths from 1 to 3000 (some requests fit one chunk, some need several); B = 300 is
    # past the longest-first limit of 256 requests
    rng = np.random.Generator(np.random.PCG64(2300 + B))
    L = rng.integers(1, 3000, size=B).astype(np.int32)
    paths, _ = random_trees(2400 + B, B, 17, 6)
    c = Case(f"ragged_hint_B{B}", L, trees=paths, seed=2500 + B)
    out, lse = c.run(prefix_len_host=L)
    c.check(out, lse, requests=None if B <= 12 else _sampled(B) + [int(np.argmax(L))])
    # a hint that understates the lengths costs balance, never correctness
    out2, lse2 = c.run(prefix_len_host=np.minimum(L, 100))
    c.check(out2, lse2, requests=[0, int(np.argmax(L))])


def _sampled(B):
    return sorted(b for b in {0, 1, B // 2, B - 1} if b < B)


def _run_as_benchmark(c):
    """Launch as the benchmark does: parent arrays read in place from pinned host memory,
    host copy of the lengths for the split plan, metadata written by the pass (checked
    bit-exactly for every request)."""
    host_parent = torch.tensor(np.array(c.parent_gpu, np.int32)).pin_memory()
    meta = _meta_outputs(c.B, c.N)
    out, lse = c.run(parent=host_parent, prefix_len_host=c.L, meta=meta)
    _assert_meta(meta, _meta_ref(c.parent_oracle, c.L))
    return out, lse


@pytest.mark.parametrize("name", ["ragged64_n33", "b64_l4096_n33", "wide32_n64"])
def test_full_size_workloads_sampled(name):
    spec = workloads.WORKLOADS[name]
    trees, _ = workloads.trees_for(spec)
    L = workloads.prefix_lengths(spec)
    c = Case(name, L, trees=trees, Hq=spec["Hq"], Hkv=spec["Hkv"], D=spec["D"],
             seed=1000 + spec["k"], k_scale=spec.get("k_scale", False))
    out, lse = _run_as_benchmark(c)
    c.check(out, lse, requests=_sampled(c.B) + [int(np.argmax(c.L))])


@pytest.mark.parametrize("B", [1, 16])
def test_long_context_paged_sampled(B):
    spec = workloads.WORKLOADS["long_paged_n33"]
    trees, _ = workloads.trees_for(spec, batch=B)
    L = workloads.prefix_lengths(spec, batch=B)
    c = Case(f"long_paged_B{B}", L, trees=trees, seed=1005, page_size=16, page_seed=3005)
    out, lse = _run_as_benchmark(c)
    c.check(out, lse, requests=_sampled(B)[:3])


@pytest.mark.parametrize("B", [2, 4, 8, 32, 64, 128])
def test_long_context_paged_batch_sweep(B):
    # the rest of the long-context sweep (batch 1..128): pools of up to 17 GB are filled
    # on the device request by request; the same seeds as the host-built B = 1, 16 cases
    spec = workloads.WORKLOADS["long_paged_n33"]
    trees, _ = workloads.trees_for(spec, batch=B)
    L = workloads.prefix_lengths(spec, batch=B)
    c = StreamedPagedCase(f"long_paged_sweep_B{B}", L, trees, seed=1005, page_size=16,
                          page_seed=3005)
    out, lse = _run_as_benchmark(c)
    rng = np.random.Generator(np.random.PCG64(7000 + B))
    extra = [int(x) for x in rng.choice(B, size=min(B, 2), replace=False)]
    c.check(out, lse, requests=sorted(set(_sampled(B)[:3] + extra)))
    c.release()


def test_streamed_case_matches_host_built_batch():
    # the streamed construction draws exactly the values of the host-built batch
    spec = workloads.WORKLOADS["long_paged_n33"]
    trees, _ = workloads.trees_for(spec, batch=2)
    L = np.array([300, 1000], np.int32)
    a = StreamedPagedCase("streamed_vs_host_s", L, trees, seed=1005, page_size=16,
                          page_seed=3005)
    b = Case("streamed_vs_host_h", L, trees=trees, seed=1005, page_size=16, page_seed=3005)
    db = b.device()
    assert np.array_equal(a.host["page_table"], b.host["page_table"])
    for key in ("q", "k", "v"):
        assert torch.equal(a.device()[key].view(torch.int16), db[key].view(torch.int16)), key
    out_a, lse_a = a.run()
    out_b, lse_b = b.run()
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


def test_full_size_through_the_batched_builder():
    # the benchmark's step: the library's batched builder writes the parent rows straight
    # into pinned host memory, the pass reads them in place and exports the metadata
    spec = workloads.WORKLOADS["b64_l4096_n33"]
    trees, _ = workloads.trees_for(spec)
    L = workloads.prefix_lengths(spec)
    c = Case("b64_batched_builder", L, trees=trees, seed=1000 + spec["k"])
    pinned = torch.empty((c.B, c.N), dtype=torch.int32).pin_memory()
    built = tv.tree_meta_build_batch(tv.PackedTrees(trees), L, c.N, parent=pinned.numpy())
    assert (built["num_nodes"] == c.N).all()
    meta = _meta_outputs(c.B, c.N)
    out, lse = c.run(parent=pinned, prefix_len_host=c.L, meta=meta)
    _assert_meta(meta, _meta_ref(c.parent_oracle, c.L))
    rng = np.random.Generator(np.random.PCG64(7100))
    reqs = sorted(set(_sampled(c.B) + [int(x) for x in rng.choice(c.B, 3, replace=False)]))
    c.check(out, lse, requests=reqs)


def test_split_pass_on_a_side_stream():
    # buffers the binding creates (outputs, split workspace) are allocated on the launch
    # stream, so a pass enqueued on a non-current stream is not overwritten by later work
    # on the current stream
    paths, _ = random_trees(2700, 4, 33, 8)
    c = Case("side_stream", [3000, 1500, 64, 2500], trees=paths, seed=2701)
    ref_out, ref_lse = c.run(num_splits=5)
    d = c.device()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        out, lse = tv.tree_verify_attn(d["q"], d["k"], d["v"], d["parent"], d["prefix_len"],
                                       3000, num_splits=5, stream=side)
        # scribble on fresh memory on the current stream meanwhile
        junk = torch.full((64 << 20,), 7, dtype=torch.uint8, device="cuda")
        del junk
        side.synchronize()
        assert np.array_equal(out.float().cpu().numpy(), ref_out)
        assert np.array_equal(lse.cpu().numpy(), ref_lse)
    torch.cuda.current_stream().wait_stream(side)


@pytest.mark.parametrize("page_size", [1, 8, 12, 32, 64, 256])
@pytest.mark.parametrize("D", [64, 128])
def test_paged_page_sizes(page_size, D):
    # power-of-two pages holding whole 1 KB load instructions take the wave-uniform page
    # lookup; 1- and 12-token pages the per-lane path; prefixes not page-aligned
    paths, _ = random_trees(2000 + page_size, 3, 33, 8)
    c = Case(f"paged_ps{page_size}_d{D}", [900, 33, 517], trees=paths, D=D,
             seed=2100 + page_size + D, page_size=page_size, page_seed=3100 + page_size)
    for splits in (0, 2):
        out, lse = c.run(num_splits=splits)
        c.check(out, lse)


@pytest.mark.parametrize("splits", [4, 8])
def test_paged_equals_contiguous_bit_for_bit(splits):
    # The paged and contiguous instantiations differ only in how a tile's rows are
    # addressed, so the same keys in either layout give the same bits (same split plan:
    # every split fits the page-table slice).  Eight splits make 320 workgroups, more than
    # one per compute unit, so the paged tiles take the vector-address form; four make 160,
    # which run two teams per workgroup and the scalar form.
    import torch
    paths, _ = random_trees(2400, 5, 33, 8)
    c = Case("paged_vs_contig", [1500, 33, 4000, 700, 2222], trees=paths, seed=2401,
             page_size=16, page_seed=3401)
    d = c.device()
    out_p, lse_p = c.run(num_splits=splits)
    table = d["page_table"].long()
    B, pages = table.shape
    k_c = d["k"][table].reshape(B, pages * 16, c.Hkv, c.D).contiguous()
    v_c = d["v"][table].reshape(B, pages * 16, c.Hkv, c.D).contiguous()
    say(c.name, "contiguous copy", {"num_splits": splits})
    out_c, lse_c = tv.tree_verify_attn(d["q"], k_c, v_c, d["parent"], d["prefix_len"],
                                       max_prefix_len=int(c.L.max()), num_splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(out_p, out_c.float().cpu().numpy().astype(np.float64))
    assert np.array_equal(lse_p, lse_c.cpu().numpy().astype(np.float64))
    c.check(out_p, lse_p)


def test_paged_small_full_with_splits():
    spec = workloads.WORKLOADS["long_paged_n33"]
    trees, _ = workloads.trees_for(spec, batch=4)
    c = Case("paged_small", [1000, 17, 400, 2048], trees=trees, seed=1905, page_size=16,
             page_seed=3905)
    for splits in (0, 1, 5):
        out, lse = c.run(num_splits=splits)
        c.check(out, lse)
