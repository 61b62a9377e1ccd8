"""Oracle: what happens after the verify pass -- TEST INFRASTRUCTURE ONLY.

Greedy acceptance on the tree and the compaction of the accepted path's KV entries, in
plain Python / numpy, sharing nothing with the HIP path.

Sources:
  [TAM] "Tree attention mask for draft-tree verification" (inferenceinterviews.com),
        "A strong answer" (the greedy walk and its tests) and "What it costs" (the
        accepted entries are moved to contiguous positions before the next step).
  [TV]  "Tree Verification" (stable-lab specdec notes), "Accepting on a Tree" (top-down
        walk, first matching child wins, a replacement token where the walk stops, a
        bonus token at a leaf) and "The Cost Side" (everything off the surviving path is
        rolled back).

Readings where the pages leave a step open (shared with the HIP path as written
specification only):
  * argmax ties go to the lowest vocabulary index; a row holding NaN returns its first
    NaN (numpy's rule);
  * children are tried in node order (the order the tree builder emits);
  * the root's own token is never checked (it is the last accepted token);
  * compaction moves the K and V rows of accepted node a_j from logical position
    L + a_j to L + j; rows at or past L + A are left as they are (rolled back: the new
    cache length is L + A).
"""
import numpy as np

from . import meta as _meta


def argmax_rows(logits):
    """Target's greedy next token after every node: argmax over the last axis, lowest
    index on ties, first NaN if a row holds one ([TAM] accept_greedy's target_argmax)."""
    x = np.asarray(logits, dtype=np.float64)
    return np.argmax(x, axis=-1).astype(np.int64)


def children(parent, node):
    """Children of ``node`` in node order."""
    return [c for c in range(len(parent)) if parent[c] == node]


def accept_greedy(parent, tokens, target_argmax):
    """Greedy walk ([TAM] "A strong answer"; [TV] "Accepting on a Tree").

    Start at the root.  At the current node the target's greedy token is emitted; then
    the first child (in node order) whose draft token equals that greedy token is
    accepted and becomes the current node.  The walk stops when no child matches (the
    emitted token is then the correction) or the node is a leaf (the emitted token is
    the bonus).

    Returns (accepted node indices, root first; emitted tokens).  len(emitted) =
    len(accepted) and ranges over 1 .. depth + 1.
    """
    parent = [int(p) for p in parent]
    _meta.validate_parent(parent)
    node, accepted, emitted = 0, [0], []
    while True:
        want = int(target_argmax[node])
        emitted.append(want)
        nxt = None
        for c in children(parent, node):
            if int(tokens[c]) == want:
                nxt = c
                break
        if nxt is None:
            return accepted, emitted
        accepted.append(nxt)
        node = nxt


def is_root_path(parent, accepted):
    """True when ``accepted`` starts at the root and each entry is a child of the one
    before it."""
    if len(accepted) == 0 or accepted[0] != 0:
        return False
    return all(0 <= accepted[j] < len(parent) and parent[accepted[j]] == accepted[j - 1]
               for j in range(1, len(accepted)))


def compact_request(k, v, prefix_len, accepted):
    """KV after acceptance ([TAM] "What it costs"; [TV] "The Cost Side").

    k, v: [T, Hkv, D] logical rows of one request (prefix, then tree nodes in node
    order).  Row L + j of the result holds the old row L + accepted[j]; every other row is
    unchanged.  Returns new arrays and the new cache length L + len(accepted).
    """
    k2, v2 = np.array(k, copy=True), np.array(v, copy=True)
    L = int(prefix_len)
    for j, a in enumerate(accepted):
        k2[L + j] = k[L + a]
        v2[L + j] = v[L + a]
    return k2, v2, L + len(accepted)
