"""Pins for the fp64 attention oracle (CPU only).

The oracle (``oracle.attn``: one dense masked softmax over the full step mask) is pinned
against things other than itself:
* brute force through an independent library routine -- ordinary causal
  ``scaled_dot_product_attention`` over each node's exact root path (``oracle.brute``) --
  on every tree with up to 6 nodes, with repeated token labels, and with rotary
  positions applied by sequential position on the path side;
* closed forms: the empty tree is single-query decoding over L+1 keys; equal scores give
  log(#allowed keys) and the mean of the allowed values;
* invariants: a chain is causal attention over its last N rows; editing a non-ancestor
  leaves a node bit-identical; relabelling permutes the outputs;
* planted mistakes: each plausible error (sibling leak, causal-over-nodes mask, lost
  prefix, parent-only mask, swapped K/V, wrong scale, sequential positions) is put into a
  copy of the oracle and must be caught by one of the pins above.
"""
import itertools

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import attn, brute, meta
from tree_attention_draft_amd import workloads

TOL = 1e-12


def all_parent_arrays(n):
    for choice in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(choice)


def labelled_inputs(rng, n, L, hq, hkv, d, n_labels=3):
    """Prefix K/V random; tree-node Q/K/V rows drawn from a small label table so that
    different histories share identical token vectors (repeated labels)."""
    lab_q = rng.standard_normal((n_labels, hq, d))
    lab_k = rng.standard_normal((n_labels, hkv, d))
    lab_v = rng.standard_normal((n_labels, hkv, d))
    labels = rng.integers(0, n_labels, size=n)
    q = lab_q[labels]
    k = np.concatenate([rng.standard_normal((L, hkv, d)), lab_k[labels]])
    v = np.concatenate([rng.standard_normal((L, hkv, d)), lab_v[labels]])
    return q, k, v


def rope(x, positions, base=10000.0):
    """Rotary embedding on the last axis (pairs (2i, 2i+1)), by integer positions."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    inv = base ** (-np.arange(0, d, 2) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]   # [T, d/2]
    shape = [len(positions)] + [1] * (x.ndim - 2) + [d // 2]
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def check_vs_brute(q, k, v, parent, L, tol=TOL, tree_fn=None):
    tree_fn = tree_fn or attn.tree_attention_request
    o1, l1 = tree_fn(q, k, v, parent, L)
    o2, l2 = brute.path_attention_request(q, k, v, parent, L)
    return max(np.abs(o1 - o2).max(), np.abs(l1 - l2).max()) <= tol


# ----------------------------------------------------------------- brute force ------
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_every_small_tree_matches_per_path_causal_attention(n):
    rng = np.random.Generator(np.random.PCG64(100 + n))
    for parent in all_parent_arrays(n):
        L = int(rng.integers(0, 5))
        q, k, v = labelled_inputs(rng, n, L, hq=4, hkv=2, d=8)
        assert check_vs_brute(q, k, v, parent, L), parent


def test_random_larger_trees_match_brute_force():
    rng = np.random.Generator(np.random.PCG64(7))
    for n, cap in [(10, 4), (33, 8), (64, 10)]:
        paths, _ = workloads.random_tree(rng, n, cap)
        parent = meta.build_from_paths(paths, 0)["parent"]
        q, k, v = labelled_inputs(rng, n, 13, hq=8, hkv=2, d=16)
        assert check_vs_brute(q, k, v, parent, 13, tol=1e-11)


def _rope_tree_run(q, k, v, parent, L, positions):
    kr = k.copy()
    kr[:L] = rope(k[:L], np.arange(L))
    kr[L:L + len(parent)] = rope(k[L:L + len(parent)], positions)
    return attn.tree_attention_request(rope(q, positions), kr, v, parent, L)


@pytest.mark.parametrize("seed", range(4))
def test_rotary_positions_prefix_plus_depth(seed):
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    trees = [meta.build_from_paths(workloads.TEN_NODE_PATHS, 0)["parent"]]
    paths, creation = workloads.random_tree(rng, 12, 4)
    trees += [meta.build_from_paths(paths, 0)["parent"], creation]
    for parent in trees:
        L = 6
        q, k, v = labelled_inputs(rng, len(parent), L, hq=2, hkv=1, d=8)
        pos = meta.meta_from_parent(parent, L)["pos"]
        o1, l1 = _rope_tree_run(q, k, v, parent, L, pos)
        o2, l2 = brute.path_attention_request(q, k, v, parent, L, rope=rope)
        assert np.abs(o1 - o2).max() <= 1e-12 and np.abs(l1 - l2).max() <= 1e-12


def test_sequential_positions_are_caught_by_rotary_pin():
    """Negative control: flattened-order positions (L + node index) must fail the pin."""
    rng = np.random.Generator(np.random.PCG64(9))
    parent = meta.build_from_paths(workloads.TEN_NODE_PATHS, 0)["parent"]
    L = 6
    q, k, v = labelled_inputs(rng, len(parent), L, hq=2, hkv=1, d=8)
    wrong = [L + i for i in range(len(parent))]
    o1, _ = _rope_tree_run(q, k, v, parent, L, wrong)
    o2, _ = brute.path_attention_request(q, k, v, parent, L, rope=rope)
    assert np.abs(o1 - o2).max() > 1e-3


# ----------------------------------------------------------------- closed forms -----
def test_empty_tree_is_single_query_decoding():
    rng = np.random.Generator(np.random.PCG64(11))
    L, hq, hkv, d = 16, 4, 2, 64
    q = rng.standard_normal((1, hq, d))
    k = rng.standard_normal((L + 1, hkv, d))
    v = rng.standard_normal((L + 1, hkv, d))
    out, lse = attn.tree_attention_request(q, k, v, [-1], L)
    for h in range(hq):
        s = (k[:, h // 2, :] @ q[0, h]) / np.sqrt(d)
        assert np.abs(out[0, h] - softmax(s) @ v[:, h // 2, :]).max() <= TOL
        assert abs(lse[0, h] - logsumexp(s)) <= TOL


def test_equal_scores_give_counting_closed_form():
    """q = 0 makes every allowed score equal: lse = log(L + depth + 1) and the output is
    the plain mean of the allowed values (prefix rows plus the node's root path)."""
    rng = np.random.Generator(np.random.PCG64(12))
    parent = meta.build_from_paths(workloads.TEN_NODE_PATHS, 0)["parent"]
    n, L, d = len(parent), 5, 4
    q = np.zeros((n, 1, d))
    k = rng.standard_normal((L + n, 1, d))
    v = rng.standard_normal((L + n, 1, d))
    out, lse = attn.tree_attention_request(q, k, v, parent, L)
    depth = [0, 1, 1, 2, 2, 2, 3, 3, 3, 4]
    for i in range(n):
        assert abs(lse[i, 0] - np.log(L + depth[i] + 1)) <= TOL
        rows = list(range(L)) + [L + j for j in brute.root_path(parent, i)]
        assert np.abs(out[i, 0] - v[rows, 0].mean(axis=0)).max() <= TOL


# ----------------------------------------------------------------- invariants -------
def test_chain_is_causal_attention_over_last_rows():
    rng = np.random.Generator(np.random.PCG64(13))
    n, L, hq, hkv, d = 6, 9, 4, 2, 16
    parent = meta.build_from_paths(workloads.chain_paths(n), L)["parent"]
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((L + n, hkv, d))
    v = rng.standard_normal((L + n, hkv, d))
    out, _ = attn.tree_attention_request(q, k, v, parent, L)
    qs = np.zeros((L + n, hq, d))
    qs[L:] = q
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(qs), t(k), t(v), is_causal=True, enable_gqa=True)[0].numpy().transpose(1, 0, 2)
    assert np.abs(out - ref[L:]).max() <= TOL


def test_non_ancestor_edits_leave_node_bit_identical():
    rng = np.random.Generator(np.random.PCG64(14))
    parent = meta.build_from_paths(workloads.TEN_NODE_PATHS, 0)["parent"]
    n, L = len(parent), 7
    q, k, v = labelled_inputs(rng, n, L, hq=2, hkv=1, d=8)
    base, base_lse = attn.tree_attention_request(q, k, v, parent, L)
    for i in range(n):
        anc = set(brute.root_path(parent, i))
        k2, v2 = k.copy(), v.copy()
        for j in range(n):
            if j not in anc:
                k2[L + j] = rng.standard_normal(k2[L + j].shape) * 100
                v2[L + j] = rng.standard_normal(v2[L + j].shape) * 100
        o, l = attn.tree_attention_request(q, k2, v2, parent, L)
        assert np.array_equal(o[i], base[i]) and np.array_equal(l[i], base_lse[i])


def test_relabelling_permutes_outputs():
    rng = np.random.Generator(np.random.PCG64(15))
    paths, creation = workloads.random_tree(rng, 20, 5)
    canon = meta.build_from_paths(paths, 0)
    # map generator (creation) index -> canonical node index via the rank paths
    gen_paths = [()] + paths
    canon_index = {p: i for i, p in enumerate(canon["paths"])}
    perm = [canon_index[p] for p in gen_paths]       # creation i -> canonical perm[i]
    n, L = 20, 4
    q, k, v = labelled_inputs(rng, n, L, hq=2, hkv=1, d=8)     # in canonical order
    out_c, lse_c = attn.tree_attention_request(q, k, v, canon["parent"], L)
    qg = q[perm]
    kg = np.concatenate([k[:L], k[L:][perm]])
    vg = np.concatenate([v[:L], v[L:][perm]])
    out_g, lse_g = attn.tree_attention_request(qg, kg, vg, creation, L)
    assert np.abs(out_g - out_c[perm]).max() <= TOL
    assert np.abs(lse_g - lse_c[perm]).max() <= TOL


# ----------------------------------------------------------------- small helpers ----
def test_bf16_decoder_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x0000, 0x8000], np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, np.inf, 0.0, -0.0]
    got = attn.bf16_bits_to_f64(bits)
    assert list(got) == want and np.signbit(got[-1])


def test_bf16_round_trip_of_generator():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.14159, 1e-40], np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    # ties to even: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1 + 2^-6
    assert list(attn.bf16_bits_to_f64(bits)[:3]) == [1.0, 1.0, 1.0 + 2 ** -6]
    assert abs(attn.bf16_bits_to_f64(bits)[3] + 3.14159) < 2 ** -6


def test_paged_gather_matches_scatter_of_contiguous_data():
    rng = np.random.Generator(np.random.PCG64(16))
    B, T, ps, hkv, d = 3, 37, 16, 2, 4
    table, n_pages = workloads.page_table(rng, B, T, ps)
    contiguous = rng.standard_normal((B, table.shape[1] * ps, hkv, d))
    pool = np.full((n_pages, ps, hkv, d), np.nan)
    for b in range(B):
        for p in range(table.shape[1]):
            pool[table[b, p]] = contiguous[b, p * ps:(p + 1) * ps]
    for b in range(B):
        assert np.array_equal(attn.gather_paged(pool, table[b], ps, T), contiguous[b, :T])


# ----------------------------------------------------------------- planted mistakes -
def _mutant(kind):
    """A copy of the oracle's attention with one plausible mistake planted."""
    def fn(q, k, v, parent, L):
        n = len(parent)
        if kind == "causal_over_nodes":
            mask = np.tril(np.ones((n, n), dtype=bool))
        elif kind == "parent_only":
            mask = np.eye(n, dtype=bool)
            for i, p in enumerate(parent):
                if p >= 0:
                    mask[i, p] = True
        elif kind == "sibling_leak":
            mask = np.array(meta.dense_mask(parent), dtype=bool)
            d = meta.meta_from_parent(parent, 0)["depth"]
            for i in range(n):
                for j in range(n):
                    if d[j] == d[i]:
                        mask[i, j] = True
        else:
            mask = np.array(meta.dense_mask(parent), dtype=bool)
        full = np.concatenate([np.ones((n, L), bool), mask], axis=1)
        if kind == "no_prefix":
            full[:, :L] = False
        kk, vv = (v, k) if kind == "swap_kv" else (k, v)
        hq, d_ = q.shape[1], q.shape[2]
        g = hq // k.shape[1]
        scale = 1.0 if kind == "no_scale" else 1.0 / np.sqrt(d_)
        out = np.zeros_like(q)
        lse = np.zeros(q.shape[:2])
        for h in range(hq):
            s = scale * (q[:, h] @ kk[:L + n, h // g].T)
            s = np.where(full, s, -np.inf)
            lse[:, h] = logsumexp(s, axis=1)
            out[:, h] = np.exp(s - lse[:, h:h + 1]) @ vv[:L + n, h // g]
        return out, lse
    return fn


@pytest.mark.parametrize("kind", ["causal_over_nodes", "parent_only", "sibling_leak",
                                  "no_prefix", "swap_kv", "no_scale"])
def test_planted_mistakes_are_caught(kind):
    rng = np.random.Generator(np.random.PCG64(17))
    parent = meta.build_from_paths(workloads.TEN_NODE_PATHS, 0)["parent"]
    q, k, v = labelled_inputs(rng, len(parent), 5, hq=2, hkv=1, d=8)
    assert check_vs_brute(q, k, v, parent, 5, tree_fn=_mutant("none"))
    assert not check_vs_brute(q, k, v, parent, 5, tree_fn=_mutant(kind))
