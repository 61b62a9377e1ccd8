"""Tree metadata in pure Python integers -- test infrastructure (see ``oracle/__init__``).

What is computed, and where the pages fix it:

* A draft candidate is a tuple of drafter ranks; rank 0 is the top guess, so ``(0, 1)`` is
  the second guess for the token that follows the top guess.  Node 0 is the root, the
  last accepted token, with the empty path.  [TAM, "A strong answer", the tree paragraph]
* Distinct paths become nodes 1.. in (length, lexicographic) order.  A candidate whose
  path minus its last rank is neither the root nor another candidate is rejected.  The
  parent of a node is the node of that shortened path; its depth is the path length
  (root 0).  [TAM, "A strong answer", build listing and tests paragraph; EBH: depth
  counts from the root, whose children sit at depth 1]
* A node sees another tree node only when that node is itself or lies on its own root
  path; alternatives on other branches are never visible.  For rank paths this is the
  prefix relation: node j is an ancestor-or-self of node i exactly when j's path is a
  prefix of i's path.  [TAM, "A strong answer", the mask paragraph; TV, "Tree Attention"]
* Position id = prefix length + depth, so siblings share a position.
  [TAM, "TL;DR" and the mask paragraph; TV, "Tree Attention"; EBH]
* Any storage order in which a parent precedes its children is valid; the meaning comes
  from the parent array alone.  [TV, "Tree Attention"; EBH]

Two derivations are kept on purpose, so that each checks the other: ``build_from_paths``
takes the ancestor relation from the path-prefix relation, ``meta_from_parent`` from the
parent array (a node's ancestor set is its parent's set plus itself).

Readings where the pages are silent (each is also listed in the design notes):
* an empty tuple or a negative rank is an invalid path (error "invalid_path");
* on a missing parent the error names the offending path's index in the *input*
  sequence (first occurrence), for the first such path in node order;
* the bitmask of node i has bit j set (LSB-first) iff node j is i or an ancestor of i;
  bits at or above N are zero.
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


def _is_prefix(a, b):
    """True when rank tuple ``a`` is a prefix of rank tuple ``b`` (``a == b`` included)."""
    return len(a) <= len(b) and b[:len(a)] == a


def _bits(rows):
    """Per row of a boolean matrix, the integer with bit j set where the row is True."""
    return [sum(1 << j for j, on in enumerate(row) if on) for row in rows]


def build_from_paths(paths, prefix_len, max_nodes=MAX_NODES):
    """Rank paths -> tree metadata.

    Returns a dict with ``parent``, ``depth``, ``pos`` (lists of int), ``bitmask`` (list of
    Python ints, one per node), ``mask`` (nested bool lists) and ``paths`` (the node order:
    ``paths[i]`` is node i's rank tuple, ``()`` for the root).  Raises :class:`TreeError`.
    """
    # distinct candidates, each remembered by the input index of its first occurrence
    seen_at = {}
    for k, p in enumerate(paths):
        seen_at.setdefault(_canonical_path(p, k), k)
    nodes = [()] + sorted(seen_at, key=lambda t: (len(t), t))
    n = len(nodes)
    if n > max_nodes:
        raise TreeError("capacity", -1, f"{n} nodes exceed the capacity of {max_nodes}")

    # parent: the node whose path is this path minus its last rank (searched for)
    parent = [-1]
    for i in range(1, n):
        shorter = nodes[i][:-1]
        hits = [j for j in range(n) if nodes[j] == shorter]
        if not hits:
            raise TreeError("missing_parent", seen_at[nodes[i]],
                            f"path {nodes[i]} (input index {seen_at[nodes[i]]}) has no "
                            f"parent {shorter}")
        parent.append(hits[0])

    depth = [len(t) for t in nodes]
    mask = [[_is_prefix(nodes[j], nodes[i]) for j in range(n)] for i in range(n)]
    return {
        "parent": parent,
        "depth": depth,
        "pos": [prefix_len + d for d in depth],
        "bitmask": _bits(mask),
        "mask": mask,
        "paths": nodes,
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


def ancestor_sets(parent):
    """Ancestor-or-self set of every node of a parent-before-child array: the root's is
    {0}; any other node's is its parent's set plus itself (the parent comes first, so its
    set is already known)."""
    sets = []
    for i, p in enumerate(parent):
        sets.append({i} if p < 0 else sets[p] | {i})
    return sets


def dense_mask(parent):
    """N x N nested lists of bools: ``mask[i][j]`` is True iff j is i or an ancestor of i."""
    parent = [int(x) for x in parent]
    validate_parent(parent)
    sets = ancestor_sets(parent)
    n = len(parent)
    return [[j in sets[i] for j in range(n)] for i in range(n)]


def meta_from_parent(parent, prefix_len):
    """Parent array (parent-before-child order) -> depth, bitmask, pos, mask."""
    parent = [int(x) for x in parent]
    validate_parent(parent)
    depth = [0] * len(parent)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
    mask = dense_mask(parent)
    return {
        "parent": parent,
        "depth": depth,
        "pos": [prefix_len + d for d in depth],
        "bitmask": _bits(mask),
        "mask": mask,
    }
