"""Pins for the rotary oracle (CPU only).

``oracle.rope`` is pinned against things other than itself:
* the complex-number form of the rotation (pair (x_i, x_{i+D/2}) as x_i + j x_{i+D/2}
  times exp(j * angle), numpy complex arithmetic), position 0 = identity, norms kept,
  rotations compose additively, and scores depend only on the position difference;
* the page's correctness condition ([TAM] probe on sibling positions, [EBH]): the fused
  tree pass (unrotated queries and tree keys rotated at L + depth, prefix keys cached
  rotated) equals an ordinary causal pass over every root path with sequential positions
  (``oracle.brute`` over ``torch`` SDPA, which rotates everything itself), on the worked
  tree, random trees, and repeated labels; positions L + node index fail it;
* after the fused compaction every cached key is rotated at its own position: ordinary
  causal attention of the last accepted node over the compacted cache equals the fused
  tree pass's output for it;
* planted mistakes (wrong sign, interleaved pairs, depth off by one) fail these pins.
"""
import numpy as np
import pytest

from oracle import accept, brute, meta, rope
from tree_attention_draft_amd import workloads

THETA = 10000.0


def labelled(rng, n, L, hq, hkv, d, n_labels=3):
    lab = rng.standard_normal((3, n_labels, max(hq, hkv), d))
    labels = rng.integers(0, n_labels, size=n)
    q = lab[0][labels][:, :hq]
    k = np.concatenate([rng.standard_normal((L, hkv, d)), lab[1][labels][:, :hkv]])
    v = np.concatenate([rng.standard_normal((L, hkv, d)), lab[2][labels][:, :hkv]])
    return q, k, v


# ------------------------------------------------------------------ the rotation ----
def complex_form_error(rotate_fn):
    """Largest difference between rotate_fn and the complex-number form of the rotation."""
    rng = np.random.Generator(np.random.PCG64(1))
    d = 16
    x = rng.standard_normal((7, 3, d))
    pos = np.array([0, 1, 2, 5, 100, 4095, 32800])
    w = THETA ** (-(2.0 * np.arange(d // 2)) / d)
    z = (x[..., :d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * w)
    return np.abs(rotate_fn(x, pos, THETA) - np.concatenate([z.real, z.imag], -1)).max()


def test_complex_form_and_basic_identities():
    assert complex_form_error(rope.rotate) < 1e-12
    rng = np.random.Generator(np.random.PCG64(1))
    d = 16
    x = rng.standard_normal((7, 3, d))
    pos = np.array([0, 1, 2, 5, 100, 4095, 32800])
    got = rope.rotate(x, pos, THETA)
    assert np.array_equal(rope.rotate(x[:1], [0], THETA), x[:1])
    assert np.allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    twice = rope.rotate(rope.rotate(x, pos, THETA), pos + 3, THETA)
    assert np.abs(twice - rope.rotate(x, 2 * pos + 3, THETA)).max() < 1e-9


def test_scores_depend_on_position_difference_only():
    rng = np.random.Generator(np.random.PCG64(2))
    q, k = rng.standard_normal((2, 64))
    for m, n in [(10, 3), (500, 200), (4100, 4096)]:
        a = rope.rotate(q[None], [m], THETA)[0] @ rope.rotate(k[None], [n], THETA)[0]
        b = rope.rotate(q[None], [m - n], THETA)[0] @ k
        assert abs(a - b) < 1e-10


# --------------------------------------------------- fused tree pass = path runs ------
def brute_rope(x, positions):
    return rope.rotate(x, positions, THETA)


def fused_vs_brute(q, k, v, parent, L):
    kc = np.array(k, copy=True)
    kc[:L] = rope.rotate(k[:L], np.arange(L), THETA)          # prefix cached rotated
    o1, l1 = rope.tree_attention_request_rope(q, kc, v, parent, L, THETA)
    o2, l2 = brute.path_attention_request(q, k, v, parent, L, rope=brute_rope)
    return max(np.abs(o1 - o2).max(), np.abs(l1 - l2).max())


@pytest.mark.parametrize("seed", range(4))
def test_fused_tree_pass_equals_per_path_runs(seed):
    rng = np.random.Generator(np.random.PCG64(50 + seed))
    trees = [meta.build_from_paths(workloads.TEN_NODE_PATHS, 0)["parent"]]
    paths, creation = workloads.random_tree(rng, 17, 5)
    trees += [meta.build_from_paths(paths, 0)["parent"], creation, [-1, 0, 1, 2, 3]]
    for parent in trees:
        L = int(rng.integers(0, 9))
        q, k, v = labelled(rng, len(parent), L, hq=4, hkv=2, d=16)
        assert fused_vs_brute(q, k, v, parent, L) < 1e-12


def test_sequential_positions_fail():
    rng = np.random.Generator(np.random.PCG64(60))
    parent = meta.build_from_paths(workloads.TEN_NODE_PATHS, 0)["parent"]
    L = 5
    q, k, v = labelled(rng, len(parent), L, hq=2, hkv=1, d=16)
    orig = rope.tree_positions
    try:
        rope.tree_positions = lambda par, Lp: Lp + np.arange(len(par))
        assert fused_vs_brute(q, k, v, parent, L) > 1e-3
    finally:
        rope.tree_positions = orig


# ------------------------------------------------------------- fused compaction ------
@pytest.mark.parametrize("seed", range(5))
def test_compacted_cache_is_rotated_at_its_positions(seed):
    rng = np.random.Generator(np.random.PCG64(70 + seed))
    L, hq, hkv, d = int(rng.integers(0, 30)), 4, 2, 16
    paths, _ = workloads.random_tree(rng, 14, 6)
    parent = meta.build_from_paths(paths, 0)["parent"]
    n = len(parent)
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((L + n, hkv, d))
    v = rng.standard_normal((L + n, hkv, d))
    k[:L] = rope.rotate(k[:L], np.arange(L), THETA)           # cache: prefix rotated
    out, lse = rope.tree_attention_request_rope(q, k, v, parent, L, THETA)
    tok = [-1] + list(rng.integers(0, 2, size=n - 1))
    am = list(rng.integers(0, 2, size=n))
    acc, _ = accept.accept_greedy(parent, tok, am)
    k2, v2, new_len = rope.compact_request_rope(k, v, L, acc, THETA)
    last = acc[-1]
    qr = rope.rotate(q[last][None], [new_len - 1], THETA)[0]   # its position: L + depth
    g = hq // hkv
    for h in range(hq):
        s = k2[:new_len, h // g] @ qr[h] / np.sqrt(d)
        m = s.max()
        w = np.exp(s - m)
        ref = (w[:, None] * v2[:new_len, h // g]).sum(0) / w.sum()
        assert np.abs(ref - out[last, h]).max() < 1e-12
        assert abs(m + np.log(w.sum()) - lse[last, h]) < 1e-12


# ------------------------------------------------------------------- planted -------
def test_planted_mistakes_fail():
    rng = np.random.Generator(np.random.PCG64(80))
    parent = meta.build_from_paths(workloads.TEN_NODE_PATHS, 0)["parent"]
    L = 4
    q, k, v = labelled(rng, len(parent), L, hq=2, hkv=1, d=16)
    orig_rotate, orig_pos = rope.rotate, rope.tree_positions

    def wrong_sign(x, positions, theta):
        return orig_rotate(x, -np.asarray(positions), theta)

    def interleaved(x, positions, theta):
        y = np.asarray(x, dtype=np.float64)
        d = y.shape[-1]
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        out = orig_rotate(y[..., perm], positions, theta)
        back = np.empty_like(out)
        back[..., perm] = out
        return back

    # any consistent rotation keeps the tree-vs-path identity, so the rotation's form is
    # caught by the complex-number pin, the position rule by the path runs
    for bad in (wrong_sign, interleaved):
        assert complex_form_error(bad) > 1e-3
    try:
        rope.tree_positions = lambda par, Lp: orig_pos(par, Lp) + 1
        assert fused_vs_brute(q, k, v, parent, L) > 1e-3
    finally:
        rope.rotate, rope.tree_positions = orig_rotate, orig_pos
