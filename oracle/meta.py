"""Tree metadata in pure Python integers -- test infrastructure (see ``oracle/__init__``).

What is computed, and where the pages fix it:

* A draft candidate is a tuple of drafter ranks; rank 0 is the top guess, so ``(0, 1)`` is
  the second guess for the token that follows the top guess.  Node 0 is the root, the
  last accepted token.  [TAM, "A strong answer", the tree paragraph and build listing]
* Distinct paths become nodes 1.. in (length, lexicographic) order.  A path whose
  one-shorter prefix is neither the root nor another path is rejected.  The parent of a
  node is the node of its one-shorter prefix; its depth is the path length (root 0).
  [TAM, "A strong answer"; EBH: first proposed tokens have depth one]
* Node i may attend to node j exactly when j is i or an ancestor of i -- never a
  sibling branch.  [TAM, "A strong answer", the mask paragraph; TV, "Tree Attention"]
* Position id = prefix length + depth, so siblings share a position.
  [TAM, "TL;DR" and the mask paragraph; TV, "Tree Attention"; EBH]
* Any storage order in which a parent precedes its children is valid; the meaning comes
  from the parent array alone.  [TV, "Tree Attention"; EBH]

Readings where the pages are silent (each is also listed in the design notes):
* an empty tuple or a negative rank is an invalid path (error "invalid_path");
* on a missing parent the error names the offending path's index in the *input*
  sequence (first occurrence), for the first such path in sorted order;
* the bitmask of node i has bit j set (LSB-first, 64 bits per word) iff node j is i or an
  ancestor of i; bits at or above N are zero.
"""

MAX_NODES = 64


class TreeError(ValueError):
    """Raised for an unusable tree.  ``code`` is one of
    ``"invalid_path"``, ``"missing_parent"``, ``"capacity"``, ``"invalid_parent"``;
    ``index`` is the offending input path (or node) index, or -1."""

    def __init__(self, code, index, msg):
        super().__init__(msg)
        self.code = code
        self.index = index


def _canonical_path(p, k):
    try:
        t = tuple(int(x) for x in p)
    except TypeError:
        raise TreeError("invalid_path", k, f"path {k} is not a sequence of ints")
    if len(t) == 0:
        raise TreeError("invalid_path", k, f"path {k} is empty (the root is implicit)")
    if any(x < 0 for x in t):
        raise TreeError("invalid_path", k, f"path {k} has a negative rank: {t}")
    return t


def ancestors_or_self(parent, i):
    """Node ids on the root path of node ``i``, from ``i`` up to the root, inclusive."""
    out = []
    j = i
    while j != -1:
        out.append(j)
        j = parent[j]
    return out


def _bitmask_from_parent(parent):
    masks = []
    for i in range(len(parent)):
        m = 0
        for j in ancestors_or_self(parent, i):
            m |= 1 << j
        masks.append(m)
    return masks


def dense_mask(parent):
    """N x N nested lists of bools: ``mask[i][j]`` is True iff j is i or an ancestor of i."""
    n = len(parent)
    rows = []
    for i in range(n):
        allowed = set(ancestors_or_self(parent, i))
        rows.append([j in allowed for j in range(n)])
    return rows


def bitmask_words(mask_int, n_words=1):
    """Split a Python-int bitmask into ``n_words`` unsigned 64-bit words, LSB first."""
    return [(mask_int >> (64 * w)) & 0xFFFFFFFFFFFFFFFF for w in range(n_words)]


def build_from_paths(paths, prefix_len, max_nodes=MAX_NODES):
    """Rank paths -> tree metadata.

    Returns a dict with ``parent``, ``depth``, ``pos`` (lists of int), ``bitmask`` (list of
    Python ints, one per node), ``mask`` (nested bool lists) and ``paths`` (the node order:
    ``paths[i]`` is node i's rank tuple, ``()`` for the root).  Raises :class:`TreeError`.
    """
    first_index = {}
    for k, p in enumerate(paths):
        t = _canonical_path(p, k)
        if t not in first_index:
            first_index[t] = k
    ordered = sorted(first_index, key=lambda t: (len(t), t))
    if len(ordered) + 1 > max_nodes:
        raise TreeError("capacity", -1,
                        f"{len(ordered) + 1} nodes exceed the capacity of {max_nodes}")
    node_of = {(): 0}
    parent = [-1]
    depth = [0]
    for t in ordered:
        up = t[:-1]
        if up not in node_of:
            raise TreeError("missing_parent", first_index[t],
                            f"path {t} (input index {first_index[t]}) has no parent {up}")
        node_of[t] = len(parent)
        parent.append(node_of[up])
        depth.append(len(t))
    return {
        "parent": parent,
        "depth": depth,
        "pos": [prefix_len + d for d in depth],
        "bitmask": _bitmask_from_parent(parent),
        "mask": dense_mask(parent),
        "paths": [()] + ordered,
    }


def validate_parent(parent):
    """Check the parent-before-child convention: ``parent[0] == -1`` and
    ``0 <= parent[i] < i`` for every other node.  Raises :class:`TreeError`."""
    n = len(parent)
    if n == 0:
        raise TreeError("invalid_parent", -1, "a tree has at least the root")
    if parent[0] != -1:
        raise TreeError("invalid_parent", 0, "node 0 must be the root (parent -1)")
    for i in range(1, n):
        if not (0 <= parent[i] < i):
            raise TreeError("invalid_parent", i,
                            f"node {i} has parent {parent[i]}; need 0 <= parent < {i}")


def meta_from_parent(parent, prefix_len):
    """Parent array (parent-before-child order) -> depth, bitmask, pos, mask."""
    parent = [int(x) for x in parent]
    validate_parent(parent)
    depth = [len(ancestors_or_self(parent, i)) - 1 for i in range(len(parent))]
    return {
        "parent": parent,
        "depth": depth,
        "pos": [prefix_len + d for d in depth],
        "bitmask": _bitmask_from_parent(parent),
        "mask": dense_mask(parent),
    }
