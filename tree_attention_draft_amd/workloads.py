"""Seeded synthetic inputs for tree-verification attention.

This module only *draws* inputs: rank-path trees, Gaussian Q/K/V, ragged prefix lengths
and page tables.  It computes none of the method's results (no masks, depths, positions
or attention), so the HIP path and the CPU oracle can both be fed from it without
sharing any of the method's arithmetic.

Recipe (stated once here, used by tests and the benchmark):
* Q, K, V ~ N(0, 1) in float32 from numpy PCG64 (host) or a seeded torch generator
  (device, for the largest shapes); bf16 workloads round those float32 values to
  bfloat16 (round to nearest even) before the device sees them.
* Trees: the worked 10-node static tree, a chain, the empty tree (root only), or random
  trees where node i's parent is drawn uniformly from the earlier nodes whose depth is
  still below a cap; a child's rank is its order of creation among its siblings.
* Ragged prefixes: L ~ Uniform{lo..hi}.  Padding beyond each request's L + N keys is
  filled with NaN so that any read of it shows up in the output.
* Paged KV: page size 16, pool = B * ceil((L + N) / 16) pages, physical ids one random
  permutation of the pool.
"""
import concurrent.futures
import os

import numpy as np

BF16_NAN_BITS = 0x7FC0

# The worked static tree of "Tree attention mask for draft-tree verification",
# rebuilt from the terms of its expected-token sum (section "What it buys"): two depth-1
# candidates (ranks 0, 1), three at depth 2, three at depth 3, one at depth 4.  Which
# depth-3 node carries the second 0.0735 term is left open by the page; the workload takes
# (0, 1, 0), i.e. the 10-node parent array -1,0,0,1,1,2,3,3,4,6.
TEN_NODE_PATHS = [(0,), (1,), (0, 0), (0, 1), (1, 0), (0, 0, 0), (0, 0, 1), (0, 1, 0),
                  (0, 0, 0, 0)]


def chain_paths(n_nodes):
    """Rank paths of a chain of top guesses with ``n_nodes`` nodes including the root."""
    return [tuple([0] * d) for d in range(1, n_nodes)]


def random_tree(rng, n_nodes, depth_cap):
    """A random tree of ``n_nodes`` nodes (root included).

    Node i (1 <= i < n) picks its parent uniformly among nodes 0..i-1 whose depth is below
    ``depth_cap``.  Returns ``(paths, creation_parent)``: the rank paths of nodes 1..n-1 in
    creation order, and the parent array in creation order (a valid parent-before-child
    labelling that is generally *not* depth-sorted).
    """
    paths = [()]
    creation_parent = [-1]
    n_children = [0]
    for i in range(1, n_nodes):
        eligible = [j for j in range(i) if len(paths[j]) < depth_cap]
        j = eligible[int(rng.integers(len(eligible)))]
        paths.append(paths[j] + (n_children[j],))
        n_children[j] += 1
        n_children.append(0)
        creation_parent.append(j)
    return paths[1:], creation_parent


def random_root_path(rng, parent):
    """Nodes from the root down to a leaf picked uniformly at random (an input for tests
    that want draft tokens agreeing with the target along one branch).  The leaf's
    ancestors are collected by climbing its parent links."""
    n = len(parent)
    has_child = [False] * n
    for c in range(1, n):
        has_child[parent[c]] = True
    leaves = [i for i in range(n) if not has_child[i]]
    node = leaves[int(rng.integers(len(leaves)))]
    up = []
    while node >= 0:
        up.append(node)
        node = parent[node]
    return up[::-1]


def random_parent(rng, n_nodes):
    """A random parent-before-child array: node i's parent drawn uniformly from 0..i-1."""
    return [-1] + [int(rng.integers(0, i)) for i in range(1, n_nodes)]


def random_distributions(rng, shape, temperature=1.0):
    """float32 next-token distributions over the last axis: a softmax of standard-normal
    logits scaled by 1 / temperature (inputs for the acceptance walks, which take
    probabilities, not logits)."""
    z = rng.standard_normal(size=shape) / temperature
    z -= z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def normal_f32(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def f32_to_bf16_bits(x, finite=False):
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.
    Finite inputs only need 32-bit arithmetic (the largest finite pattern plus the rounding
    increment stays below 2**32); NaN maps to the canonical bfloat16 NaN.  ``finite=True``
    skips the NaN scan for data known to be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r >>= np.uint32(16)
    bits = r.astype(np.uint16)
    if not finite:
        nan = np.isnan(x)
        if nan.any():
            bits[nan] = BF16_NAN_BITS
    return bits


def bf16_bits_to_f32(bits):
    """bfloat16 bits -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def ragged_lengths(rng, batch, lo, hi):
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def page_table(rng, batch, tokens_per_seq, page_size):
    """[B, pages_per_seq] int32 physical page ids: one random permutation of the pool."""
    pages_per_seq = -(-tokens_per_seq // page_size)
    perm = rng.permutation(batch * pages_per_seq).astype(np.int32)
    return perm.reshape(batch, pages_per_seq), batch * pages_per_seq


# ---------------------------------------------------------------------------------------
# Named workloads.  Seeds: tensors 1000+k, trees 2000+k, page tables 3000+k.
# ---------------------------------------------------------------------------------------
WORKLOADS = {
    # single request, the worked 10-node tree, L=16, one head, D=64, fp32
    "tree10_f32": dict(k=1, B=1, L=16, Hq=1, Hkv=1, D=64, dtype="f32", tree="tree10"),
    "empty_f32": dict(k=1, B=1, L=16, Hq=1, Hkv=1, D=64, dtype="f32", tree="empty"),
    "chain5_f32": dict(k=1, B=1, L=16, Hq=1, Hkv=1, D=64, dtype="f32", tree="chain5"),
    # batch 8, Llama-3-8B attention shape, L=2048
    "llama8b_tree10": dict(k=2, B=8, L=2048, Hq=32, Hkv=8, D=128, dtype="bf16",
                           tree="tree10"),
    "llama8b_chain5": dict(k=2, B=8, L=2048, Hq=32, Hkv=8, D=128, dtype="bf16",
                           tree="chain5"),
    # batch 64, ragged prefixes U[512, 8192], N=33 random trees capped at depth 8
    "ragged64_n33": dict(k=3, B=64, L=(512, 8192), Hq=32, Hkv=8, D=128, dtype="bf16",
                         tree="random", N=33, cap=8),
    # batch 64, L=4096, N=33 random trees (the throughput workload)
    "b64_l4096_n33": dict(k=6, B=64, L=4096, Hq=32, Hkv=8, D=128, dtype="bf16",
                          tree="random", N=33, cap=8),
    # batch 32, wide trees N=64 depth <= 10, 70B-like 64q/8kv, K scaled by 1/sqrt(D)
    "wide32_n64": dict(k=4, B=32, L=4096, Hq=64, Hkv=8, D=128, dtype="bf16",
                       tree="random", N=64, cap=10, k_scale=True),
    # long context, paged KV, page 16, L=32768, N=33; batch swept 1..128 (16 headline)
    "long_paged_n33": dict(k=5, B=16, L=32768, Hq=32, Hkv=8, D=128, dtype="bf16",
                           tree="random", N=33, cap=8, paged=16),
}


def trees_for(spec, batch=None):
    """Per-request rank paths for a workload: list of B path lists (and creation
    parents for random trees, else None)."""
    B = spec["B"] if batch is None else batch
    t = spec["tree"]
    if t == "tree10":
        return [list(TEN_NODE_PATHS) for _ in range(B)], None
    if t == "chain5":
        return [chain_paths(5) for _ in range(B)], None
    if t == "empty":
        return [[] for _ in range(B)], None
    rng = np.random.Generator(np.random.PCG64(2000 + spec["k"]))
    paths, creation = [], []
    for _ in range(B):
        p, c = random_tree(rng, spec["N"], spec["cap"])
        paths.append(p)
        creation.append(c)
    return paths, creation


def prefix_lengths(spec, batch=None):
    B = spec["B"] if batch is None else batch
    L = spec["L"]
    if isinstance(L, tuple):
        rng = np.random.Generator(np.random.PCG64(4000 + spec["k"]))
        return ragged_lengths(rng, B, L[0], L[1])
    return np.full(B, L, dtype=np.int32)


def request_tensors(seed, b, n_nodes, prefix_len, hq, hkv, d, k_scale=False):
    """float32 Q [N, Hq, D] and logical K, V [L + N, Hkv, D] of request ``b``.

    Every request draws from its own PCG64 stream (seeded with ``(seed, b)``), so any
    request can be regenerated alone.  ``k_scale`` multiplies K by 1/sqrt(D).
    """
    rng = np.random.Generator(np.random.PCG64([seed, b]))
    q = normal_f32(rng, (n_nodes, hq, d))
    k = normal_f32(rng, (prefix_len + n_nodes, hkv, d))
    v = normal_f32(rng, (prefix_len + n_nodes, hkv, d))
    if k_scale:
        k *= np.float32(1.0 / np.sqrt(d))
    return q, k, v


def encode(x, dtype):
    """Storage form of finite float32 values: bf16 bits (uint16) or float32 itself."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x, finite=True)
    return np.ascontiguousarray(x, np.float32)


def nan_fill(shape, dtype):
    if dtype == "bf16":
        return np.full(shape, BF16_NAN_BITS, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=np.float32)


def build_batch(seed, prefix_lens, n_nodes, hq, hkv, d, dtype, k_scale=False, page_size=0,
                page_seed=None):
    """Host arrays for one batch.

    Returns a dict with ``q`` [B, N, Hq, D] and either contiguous ``k``, ``v``
    [B, max L + N, Hkv, D] (NaN beyond each request's L + N) or, when ``page_size`` > 0,
    pools ``k``, ``v`` [pages, page_size, Hkv, D] plus ``page_table`` [B, pages_per_seq]
    (slots past a request's L + N are NaN).  Values are uint16 bf16 bits or float32.
    """
    B = len(prefix_lens)
    Lmax = int(max(prefix_lens)) if B else 0
    S = Lmax + n_nodes
    q = np.empty((B, n_nodes, hq, d), np.uint16 if dtype == "bf16" else np.float32)
    out = {"q": q, "prefix_len": np.asarray(prefix_lens, np.int32)}
    if page_size:
        prng = np.random.Generator(np.random.PCG64(page_seed))
        table, n_pages = page_table(prng, B, S, page_size)
        kpool = nan_fill((n_pages, page_size, hkv, d), dtype)
        vpool = nan_fill((n_pages, page_size, hkv, d), dtype)
        out.update(k=kpool, v=vpool, page_table=table, page_size=page_size)
    else:
        kc = nan_fill((B, S, hkv, d), dtype)
        vc = nan_fill((B, S, hkv, d), dtype)
        out.update(k=kc, v=vc)
    def fill(b):
        L = int(prefix_lens[b])
        qb, kb, vb = request_tensors(seed, b, n_nodes, L, hq, hkv, d, k_scale)
        q[b] = encode(qb, dtype)
        kb, vb = encode(kb, dtype), encode(vb, dtype)
        if page_size:
            T = L + n_nodes
            for pi in range(-(-T // page_size)):
                lo, hi = pi * page_size, min(T, (pi + 1) * page_size)
                out["k"][table[b, pi], :hi - lo] = kb[lo:hi]
                out["v"][table[b, pi], :hi - lo] = vb[lo:hi]
        else:
            out["k"][b, :L + n_nodes] = kb
            out["v"][b, :L + n_nodes] = vb

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, range(B)))
    return out
