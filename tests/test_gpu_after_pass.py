"""GPU parity of the after-pass entry points against ``oracle.accept``: the target's greedy
token per node (bit-exact, ties and NaN included), the greedy walk (bit-exact) and the
accepted path's KV compaction (bit-exact bytes, contiguous and paged, invalid lists left
untouched).  Everything goes through the C ABI."""
import numpy as np
import pytest

import tree_attention_draft_amd as tv
from oracle import accept as oacc
from oracle import meta as ometa
from tree_attention_draft_amd import workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print("[after-pass]", *a, flush=True)


def random_parents(seed, B, N, cap=8):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(B):
        paths, _ = workloads.random_tree(rng, N, cap)
        out.append(ometa.build_from_paths(paths, 0)["parent"])
    return out


def to_dev(x, dtype):
    import torch
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(np.asarray(x, np.float32).copy(), finite=False)
        return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.asarray(x, np.float32)).cuda()


def dev_values(t):
    return t.float().cpu().numpy().astype(np.float64)


# ------------------------------------------------------------------- argmax + walk ---
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 1000, 1024, 32003])
def test_argmax_and_walk_bit_exact(dtype, V):
    import torch
    B, N = 3, 33
    say("argmax+walk", dtype, f"B={B} N={N} V={V}")
    rng = np.random.Generator(np.random.PCG64(V))
    x = rng.standard_normal((B, N, V)).astype(np.float32)
    # ties: duplicate the row max at a later index in some rows; constant rows; -inf rows
    for n in range(0, N, 5):
        r = x[0, n]
        if V > 1:
            r[V // 2] = r.max()
    x[1, 3, :] = 0.25
    x[1, 4, :] = -np.inf
    if V > 9:              # zero is the max, -0 comes first: equal values, lowest index wins
        x[0, 2, :] = -1.0
        x[0, 2, 5] = -0.0
        x[0, 2, 9] = 0.0
        x[0, 3, :] = -2.0  # max only in the last element
        x[0, 3, V - 1] = 1.0
    if V > 3:
        x[2, 7, 2] = np.nan            # first NaN wins
        x[2, 7, V - 1] = np.nan
    logits = to_dev(x, dtype)
    parents = random_parents(700 + V, B, N)
    vocab = min(V, 4)
    tokens = [[-1] + list(rng.integers(0, vocab, size=N - 1)) for _ in range(B)]
    # make the greedy tokens small integers too so that the walk goes deep
    xs = dev_values(logits)
    par_d = torch.tensor(np.array(parents, np.int32)).cuda()
    tok_d = torch.tensor(np.array(tokens, np.int32)).cuda()
    target, acc, em, na = tv.tree_accept_greedy(logits, tok_d, par_d)
    torch.cuda.synchronize()
    want = oacc.argmax_rows(xs)
    assert np.array_equal(target.cpu().numpy(), want)
    for b in range(B):
        a_ref, e_ref = oacc.accept_greedy(parents[b], tokens[b], want[b])
        n = int(na[b])
        assert n == len(a_ref)
        assert acc[b, :n].tolist() == a_ref and em[b, :n].tolist() == e_ref
        assert (acc[b, n:] == -1).all() and (em[b, n:] == -1).all()


def test_walk_goes_deep_with_matching_logits():
    import torch
    B, N, V = 4, 33, 64
    parents = random_parents(31, B, N)
    rng = np.random.Generator(np.random.PCG64(32))
    tokens = [[-1] + list(rng.integers(0, V, size=N - 1)) for _ in range(B)]
    # the target agrees with the draft along one random root-to-leaf path per request
    x = rng.standard_normal((B, N, V)).astype(np.float32)
    for b in range(B):
        path = workloads.random_root_path(rng, list(parents[b]))
        for u, c in zip(path, path[1:]):
            x[b, u, tokens[b][c]] = 50.0
    logits = to_dev(x, "f32")
    target, acc, em, na = tv.tree_accept_greedy(
        logits, torch.tensor(np.array(tokens, np.int32)).cuda(),
        torch.tensor(np.array(parents, np.int32)).cuda())
    torch.cuda.synchronize()
    want = oacc.argmax_rows(x)
    for b in range(B):
        a_ref, e_ref = oacc.accept_greedy(parents[b], tokens[b], want[b])
        assert int(na[b]) == len(a_ref) >= 2
        assert acc[b, :len(a_ref)].tolist() == a_ref and em[b, :len(e_ref)].tolist() == e_ref


def test_argmax_vocab_of_llama3_sampled():
    import torch
    B, N, V = 2, 33, 128256
    rng = np.random.Generator(np.random.PCG64(5))
    x = (rng.standard_normal((B, N, V)) * 3).astype(np.float32)
    logits = to_dev(x, "bf16")
    parents = random_parents(5, B, N)
    tokens = [[-1] + list(rng.integers(0, V, size=N - 1)) for _ in range(B)]
    target, *_ = tv.tree_accept_greedy(logits, torch.tensor(np.array(tokens, np.int32)).cuda(),
                                       torch.tensor(np.array(parents, np.int32)).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(target.cpu().numpy(), oacc.argmax_rows(dev_values(logits)))


# ------------------------------------------------------------------------ compaction ---
def kv_case(seed, prefix, N, Hkv, D, dtype, page_size=0):
    """Host K/V (values the device sees, as float64) plus the device tensors."""
    import torch
    L = np.asarray(prefix, np.int32)
    host = workloads.build_batch(seed, L, N, 1, Hkv, D, dtype, page_size=page_size,
                                 page_seed=seed + 1)
    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    k, v = up(host["k"]), up(host["v"])
    pt = torch.from_numpy(host["page_table"]).cuda() if page_size else None
    return host, L, k, v, pt


def logical_rows(arr, host, b, T, page_size):
    if page_size:
        from oracle import attn as oattn
        return oattn.gather_paged(arr, host["page_table"][b], page_size, T)
    return arr[b, :T]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("page_size", [0, 16])
def test_compaction_bit_exact(dtype, D, page_size):
    import torch
    B, N, Hkv = 5, 33, 4
    prefix = [40, 0, 17, 300, 5]
    say("compact", dtype, f"D={D} paged={page_size}")
    host, L, k, v, pt = kv_case(1600 + D + page_size, prefix, N, Hkv, D, dtype, page_size)
    parents = random_parents(41 + D, B, N)
    rng = np.random.Generator(np.random.PCG64(D + page_size))
    # accepted lists: real greedy walks (random tokens), one full root-to-leaf path, and a
    # deliberately invalid list that must leave its request untouched
    lists = []
    for b in range(B):
        tok = [-1] + list(rng.integers(0, 2, size=N - 1))
        am = list(rng.integers(0, 2, size=N))
        lists.append(oacc.accept_greedy(parents[b], tok, am)[0])
    leaf = max(range(N), key=lambda i: ometa.meta_from_parent(parents[1], 0)["depth"][i])
    path = [leaf]
    while path[-1] != 0:
        path.append(parents[1][path[-1]])
    lists[1] = path[::-1]
    lists[3] = [0, 5, 2] if parents[3][5] != 0 or parents[3][2] != 5 else [0, 9, 1]
    acc = np.full((B, N), -1, np.int32)
    na = np.zeros(B, np.int32)
    for b, l in enumerate(lists):
        acc[b, :len(l)] = l
        na[b] = len(l)
    before_k = k.clone()
    before_v = v.clone()
    new_len, status = tv.tree_kv_compact(
        k, v, torch.from_numpy(L).cuda(), int(L.max()), torch.tensor(np.array(parents, np.int32)).cuda(),
        torch.from_numpy(acc).cuda(), torch.from_numpy(na).cuda(), page_table=pt,
        page_size=page_size)
    torch.cuda.synchronize()
    kb = k.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
    vb = v.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
    k0 = before_k.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
    v0 = before_v.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
    for b in range(B):
        T = int(L[b]) + N
        valid = oacc.is_root_path(parents[b], lists[b])
        assert int(status[b]) == (0 if valid else 1)
        assert int(new_len[b]) == int(L[b]) + (len(lists[b]) if valid else 0)
        src_k, src_v = logical_rows(k0, host, b, T, page_size), logical_rows(v0, host, b, T, page_size)
        if valid:
            ref_k, ref_v, _ = oacc.compact_request(src_k, src_v, int(L[b]), lists[b])
        else:
            ref_k, ref_v = src_k, src_v
        got_k, got_v = logical_rows(kb, host, b, T, page_size), logical_rows(vb, host, b, T, page_size)
        assert np.array_equal(got_k, ref_k) and np.array_equal(got_v, ref_v), b
    # nothing outside the requests' logical rows changed (contiguous padding / free pages)
    if not page_size:
        for b in range(B):
            T = int(L[b]) + N
            assert np.array_equal(kb[b, T:], k0[b, T:]) and np.array_equal(vb[b, T:], v0[b, T:])


def test_prepared_calls_match_the_plain_calls():
    # arguments marshalled once, calls repeated with the inputs changed in place: outputs
    # equal to the plain calls' each time (greedy, stochastic, compaction)
    import torch
    B, N, V = 6, 17, 3001
    parents = random_parents(880, B, N)
    par = torch.tensor(np.array(parents, np.int32), device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(881)
    logits = torch.randn((B, N, V), generator=g, device="cuda").to(torch.bfloat16)
    tok = torch.randint(0, V, (B, N), generator=g, device="cuda", dtype=torch.int32)
    greedy = tv.prepare_tree_accept_greedy(logits, tok, par)
    p = torch.softmax(torch.randn((B, N, V), generator=g, device="cuda"), -1)
    q = torch.softmax(torch.randn((B, N, V), generator=g, device="cuda"), -1)
    u = torch.rand((B, N), generator=g, device="cuda", dtype=torch.float64)
    stoch = tv.prepare_tree_accept_stochastic(p, q, tok, par, u)
    for rep in range(2):
        if rep:  # new inputs, same storage
            logits.copy_(torch.randn((B, N, V), generator=g, device="cuda").to(torch.bfloat16))
            p.copy_(torch.softmax(torch.randn((B, N, V), generator=g, device="cuda"), -1))
            u.copy_(torch.rand((B, N), generator=g, device="cuda", dtype=torch.float64))
        want = tv.tree_accept_greedy(logits, tok, par)
        got = greedy()
        want_s = tv.tree_accept_stochastic(p, q, tok, par, u)
        got_s = stoch()
        torch.cuda.synchronize()
        for a, b in zip(got + got_s, want + want_s):
            assert torch.equal(a, b), rep

    # compaction: the same accepted lists applied to two copies of a cache
    L, Hkv, D = 300, 4, 128
    k = torch.randn((B, L + N, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, L + N, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    k2, v2 = k.clone(), v.clone()
    pl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    _, acc, _, na = greedy.result
    comp = tv.prepare_tree_kv_compact(k2, v2, pl, L, par, acc, na)
    nl, st = tv.tree_kv_compact(k, v, pl, L, par, acc, na)
    nl2, st2 = comp()
    torch.cuda.synchronize()
    assert torch.equal(nl, nl2) and torch.equal(st, st2)
    assert torch.equal(k, k2) and torch.equal(v, v2)
