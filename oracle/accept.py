"""Oracle: what happens after the verify pass -- TEST INFRASTRUCTURE ONLY.

Greedy acceptance on the tree and the compaction of the accepted path's KV entries, in
plain Python / numpy, sharing nothing with the HIP path.

Sources:
  [TAM] "Tree attention mask for draft-tree verification" (inferenceinterviews.com),
        "A strong answer" (the greedy walk and its tests) and "What it costs" (before
        the next step the accepted nodes' cache entries are packed into consecutive
        positions).
  [TV]  "Tree Verification" (stable-lab specdec notes), "Accepting on a Tree" (top-down
        walk, first matching child wins, a replacement token where the walk stops, a
        bonus token at a leaf) and "The Cost Side" (cache entries of rejected branches
        are discarded).

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
    index on ties, first NaN if a row holds one ([TAM] "A strong answer": the walk
    compares draft tokens with the target's greedy choices)."""
    x = np.asarray(logits, dtype=np.float64)
    return np.argmax(x, axis=-1).astype(np.int64)


def child_table(parent):
    """For every node, the list of its children in ascending node order."""
    table = [[] for _ in parent]
    for c in range(1, len(parent)):
        table[parent[c]].append(c)
    return table


def accept_greedy(parent, draft, greedy_after):
    """Greedy walk ([TAM] "A strong answer"; [TV] "Accepting on a Tree").

    ``draft[i]``: the draft token of node i (node 0's is never read); ``greedy_after[i]``:
    the target's greedy token for the position after node i.

    Start at the root.  At the current node the target's greedy token is emitted; then
    the first child (in node order) whose draft token equals that greedy token is
    accepted and becomes the current node.  The walk stops when no child matches (the
    emitted token is then the correction) or the node is a leaf (the emitted token is
    the bonus).  Every step goes one level deeper, so there are at most N steps.

    Returns (accepted node indices, root first; emitted tokens).  len(emitted) =
    len(accepted) and ranges over 1 .. depth + 1.
    """
    parent = [int(p) for p in parent]
    _meta.validate_parent(parent)
    table = child_table(parent)
    accepted, emitted = [0], []
    for _ in range(len(parent)):
        here = accepted[-1]
        greedy = int(greedy_after[here])
        emitted.append(greedy)
        matching = [c for c in table[here] if int(draft[c]) == greedy]
        if not matching:
            break
        accepted.append(matching[0])
    return accepted, emitted


def is_root_path(parent, accepted):
    """True when ``accepted`` is a root path of the tree: 1 <= len <= N, it starts at the
    root, every entry is a node index, and each entry is a child of the one before it."""
    n = len(parent)
    if not 1 <= len(accepted) <= n or accepted[0] != 0:
        return False
    for prev, cur in zip(accepted, accepted[1:]):
        if not (0 <= cur < n) or parent[cur] != prev:
            return False
    return True


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
