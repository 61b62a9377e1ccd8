"""GPU parity of the fused rotary embedding against ``oracle.rope``: queries and tree keys
handed over unrotated and rotated inside the attention kernels at L + depth (prefix keys
cached rotated), on every kernel path (MFMA with and without the shared remainder tile and
node chunks, VALU in fp32 and bf16), with key splits, paged KV and long positions; and the
compaction that stores accepted keys rotated at their new positions.  Attention tolerances
as for the plain pass; compacted keys within one bf16 rounding (bf16) or 1e-5 (fp32) of
the fp64 rotation, values and untouched rows bit-exact."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
import tree_attention_draft_amd as tv  # noqa: E402
from oracle import accept as oacc  # noqa: E402
from oracle import attn as oattn  # noqa: E402
from oracle import meta as ometa  # noqa: E402
from oracle import rope as orope  # noqa: E402
from tree_attention_draft_amd import workloads  # noqa: E402

from gpu_cases import Case, say  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TEN = list(workloads.TEN_NODE_PATHS)


def random_trees(seed, B, n, cap):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [workloads.random_tree(rng, n, cap)[0] for _ in range(B)]


# ------------------------------------------------------------------ attention ----------
@pytest.mark.parametrize("theta", [10000.0, 500000.0])
def test_rope_mfma_n33_ragged_prefixes(theta):
    # prefixes chosen so the tree keys start inside a tile, on a tile edge, on a window
    # edge, and at 0
    L = [0, 31, 32, 63, 64, 100, 1000, 2047]
    c = Case("rope_n33", L, trees=random_trees(61, len(L), 33, 8), seed=1961)
    out, lse = c.run(rope_theta=theta)
    c.check(out, lse)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("hq,hkv,n", [(32, 8, 10), (16, 8, 17), (8, 8, 64), (64, 8, 64)])
def test_rope_mfma_shapes(D, hq, hkv, n):
    L = [5, 777, 96]
    c = Case(f"rope_{hq}_{hkv}_n{n}_d{D}", L, trees=random_trees(62 + n, 3, n, 10), Hq=hq,
             Hkv=hkv, D=D, seed=1962 + n)
    out, lse = c.run(rope_theta=10000.0)
    c.check(out, lse)


@pytest.mark.parametrize("splits", [2, 7])
def test_rope_with_key_splits(splits):
    L = [300, 4000, 58, 1029]
    c = Case("rope_splits", L, trees=random_trees(63, 4, 33, 8), seed=1963)
    out, lse = c.run(rope_theta=10000.0, num_splits=splits)
    c.check(out, lse)


@pytest.mark.parametrize("dtype,hq,hkv,D,tree", [("f32", 1, 1, 64, "tree10"),
                                                 ("f32", 8, 2, 128, "tree10"),
                                                 ("bf16", 1, 1, 64, "chain5"),
                                                 ("bf16", 4, 4, 128, "tree10")])
def test_rope_valu(dtype, hq, hkv, D, tree):
    paths = TEN if tree == "tree10" else workloads.chain_paths(5)
    c = Case(f"rope_valu_{dtype}", [16, 0, 70], trees=paths, Hq=hq, Hkv=hkv, D=D,
             dtype=dtype, seed=1964)
    out, lse = c.run(rope_theta=10000.0, path="valu")
    c.check(out, lse)


def test_rope_long_positions_paged():
    spec = workloads.WORKLOADS["long_paged_n33"]
    trees, _ = workloads.trees_for(spec, batch=2)
    c = Case("rope_long_paged", [32768, 20001], trees=trees, seed=1965, page_size=16,
             page_seed=3965)
    out, lse = c.run(rope_theta=500000.0)
    c.check(out, lse)


def test_rope_full_size_sampled():
    spec = workloads.WORKLOADS["b64_l4096_n33"]
    trees, _ = workloads.trees_for(spec)
    c = Case("rope_b64_l4096_n33", workloads.prefix_lengths(spec), trees=trees,
             seed=1000 + spec["k"])
    out, lse = c.run(rope_theta=500000.0)
    c.check(out, lse, requests=[0, 1, 32, 63])


def test_rope_off_is_the_plain_pass():
    c = Case("rope_off", [40, 1000], trees=random_trees(66, 2, 33, 8), seed=1966)
    o1, l1 = c.run()
    o2, l2 = c.run(rope_theta=0.0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------------ compaction ---------
def kv_case(seed, prefix, N, Hkv, D, dtype, page_size=0):
    L = np.asarray(prefix, np.int32)
    host = workloads.build_batch(seed, L, N, 1, Hkv, D, dtype, page_size=page_size,
                                 page_seed=seed + 1)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    pt = torch.from_numpy(host["page_table"]).cuda() if page_size else None
    return host, L, up(host["k"]), up(host["v"]), pt


def rows(arr, host, b, T, page_size):
    if page_size:
        return oattn.gather_paged(arr, host["page_table"][b], page_size, T)
    return arr[b, :T]


def values(bits, dtype):
    return oattn.bf16_bits_to_f64(bits) if dtype == "bf16" else bits.view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("page_size", [0, 16])
def test_rope_compaction(dtype, D, page_size):
    B, N, Hkv, theta = 5, 33, 4, 10000.0
    prefix = [40, 0, 17, 30000, 5]
    say("rope compact", dtype, f"D={D} paged={page_size}")
    host, L, k, v, pt = kv_case(2600 + D + page_size, prefix, N, Hkv, D, dtype, page_size)
    rng = np.random.Generator(np.random.PCG64(D + page_size + 7))
    parents = []
    lists = []
    for b in range(B):
        paths, _ = workloads.random_tree(rng, N, 8)
        par = ometa.build_from_paths(paths, 0)["parent"]
        parents.append(par)
        tok = [-1] + list(rng.integers(0, 2, size=N - 1))
        lists.append(oacc.accept_greedy(par, tok, list(rng.integers(0, 2, size=N)))[0])
    lists[3] = [0, 9, 1] if parents[3][9] != 0 or parents[3][1] != 9 else [0, 5, 2]  # invalid
    acc = np.full((B, N), -1, np.int32)
    na = np.zeros(B, np.int32)
    for b, lst in enumerate(lists):
        acc[b, :len(lst)] = lst
        na[b] = len(lst)
    ibits = torch.int16 if dtype == "bf16" else torch.int32
    k0 = k.view(ibits).cpu().numpy().copy()
    v0 = v.view(ibits).cpu().numpy().copy()
    new_len, status = tv.tree_kv_compact(
        k, v, torch.from_numpy(L).cuda(), int(L.max()),
        torch.tensor(np.array(parents, np.int32)).cuda(), torch.from_numpy(acc).cuda(),
        torch.from_numpy(na).cuda(), page_table=pt, page_size=page_size, rope_theta=theta)
    torch.cuda.synchronize()
    kb = k.view(ibits).cpu().numpy()
    vb = v.view(ibits).cpu().numpy()
    for b in range(B):
        T = int(L[b]) + N
        valid = oacc.is_root_path(parents[b], lists[b])
        assert int(status[b]) == (0 if valid else 1)
        A = len(lists[b]) if valid else 0
        assert int(new_len[b]) == int(L[b]) + A
        src_k, src_v = rows(k0, host, b, T, page_size), rows(v0, host, b, T, page_size)
        got_k, got_v = rows(kb, host, b, T, page_size), rows(vb, host, b, T, page_size)
        if not valid:
            assert np.array_equal(got_k, src_k) and np.array_equal(got_v, src_v)
            continue
        ref_k, ref_v, _ = orope.compact_request_rope(values(src_k, dtype), values(src_v, dtype),
                                                     int(L[b]), lists[b], theta)
        Lb = int(L[b])
        # values and every key row outside [L, L + A) bit-exact
        _, want_v_bits, _ = oacc.compact_request(src_k, src_v, Lb, lists[b])
        assert np.array_equal(got_v, want_v_bits)
        outside = [t for t in range(T) if not Lb <= t < Lb + A]
        assert np.array_equal(got_k[outside], src_k[outside])
        # rotated keys: one rounding of the output type away from the fp64 rotation
        gk = values(got_k[Lb:Lb + A], dtype)
        rk = ref_k[Lb:Lb + A]
        pair = np.sqrt(rk[..., :D // 2] ** 2 + rk[..., D // 2:] ** 2)
        pair = np.concatenate([pair, pair], -1)
        bound = (2.0 ** -8 * np.abs(rk) + 1e-5 * pair) if dtype == "bf16" else 1e-5 + 0 * rk
        err = np.abs(gk - rk)
        assert (err <= bound).all(), (b, float(err.max()))
        say("rope compact", f"b={b} A={A} max_err={float(err.max()):.2e}")
