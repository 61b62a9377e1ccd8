"""Oracle: rotary position embedding at tree positions -- TEST INFRASTRUCTURE ONLY.

numpy float64, sharing nothing with the HIP path.

Sources:
  [TAM] "Tree attention mask for draft-tree verification" (inferenceinterviews.com),
        "What interviewers probe next" (siblings share a position: rotary embedding must
        rotate a node as if it sat at its own depth) and "Common mistakes" (numbering the
        flattened nodes 0, 1, 2, ... as positions breaks rotary embeddings); "What it
        costs" (the tree's cache rows sit in node order; the accepted ones are packed
        together afterwards).
  [EBH] "Encode branch histories in masks and positions": positional features follow the
        model's position semantics (depth), not the flattened storage order.

Readings where the pages leave a step open (shared with the HIP path as written
specification only):
  * node i's query and key are rotated at position L + depth(i);
  * the rotary form is the rotate-half one: feature pairs (i, i + D/2), i < D/2, turn by
    angle pos * theta^(-2i/D), i.e. x_i + j x_{i+D/2} is multiplied by exp(j * angle);
  * in the fused form the caller hands over unrotated queries and unrotated tree keys,
    while the cached prefix keys are already rotated at their own positions; compaction
    then stores accepted node a_j's key rotated at L + j (= L + depth(a_j)), so after it
    every cached key is rotated at its position.
"""
import numpy as np

from . import accept as _accept
from . import attn as _attn
from . import meta as _meta


def inv_freq(d, theta):
    """theta^(-2i/d) for i < d/2 (float64)."""
    return float(theta) ** (-(2.0 * np.arange(d // 2)) / d)


def rotate(x, positions, theta):
    """Rotate-half rotary embedding of x [T, ..., D] at integer positions [T]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq(d, theta)[None, :]
    shape = [len(positions)] + [1] * (x.ndim - 2) + [h]
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def tree_positions(parent, prefix_len):
    """L + depth(i) for every node ([TAM] probe on sibling positions)."""
    return np.asarray(_meta.meta_from_parent(list(parent), int(prefix_len))["pos"])


def tree_attention_request_rope(q, k, v, parent, prefix_len, theta, sm_scale=None):
    """Tree attention of one request with the rotation fused in: q [N, Hq, D] and the tree
    keys k[L .. L+N) are unrotated and are rotated here at L + depth; the prefix keys
    k[:L] are taken as already rotated.  Returns (out, lse) like ``attn``."""
    L = int(prefix_len)
    n = len(parent)
    pos = tree_positions(parent, L)
    kr = np.array(k, dtype=np.float64, copy=True)
    kr[L:L + n] = rotate(kr[L:L + n], pos, theta)
    return _attn.tree_attention_request(rotate(q, pos, theta), kr, v, parent, L,
                                        sm_scale=sm_scale)


def compact_request_rope(k, v, prefix_len, accepted, theta):
    """Compaction with the rotation fused in: accepted node a_j's key, unrotated in the
    tree rows, is stored at L + j rotated at position L + j; values move unchanged."""
    k2, v2, new_len = _accept.compact_request(k, v, prefix_len, accepted)
    L = int(prefix_len)
    A = len(accepted)
    k2[L:L + A] = rotate(k2[L:L + A], L + np.arange(A), theta)
    return k2, v2, new_len
