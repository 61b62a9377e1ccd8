"""Oracle: tree-budget arithmetic -- TEST INFRASTRUCTURE ONLY.

How many nodes a step can afford at a given batch, what a tree is worth under greedy
verification, and which static tree of a given size is worth the most, in plain Python
floats (IEEE double), sharing nothing with the library's host C++ code.

Sources:
  [TAM] "Tree attention mask for draft-tree verification" (inferenceinterviews.com),
        "What it buys" (reach probability of a node = product of the probabilities of
        the ranks on its path; expected tokens per step = 1 + the sum over nodes) and
        "What it costs" (B x N tokens per step against the ridge of a bandwidth-bound
        decode step; break-even batch = ridge / N; the tree narrows to a chain, then to
        the root alone, as B x N nears the ridge).
  [TV]  "Tree Verification" (stable-lab specdec notes), "The Cost Side" (a node's expected
        contribution is its path product; spend the node budget where the acceptance mass
        is).

Readings where the pages leave a step open (shared with the library as written
specification only):
  * a node's rank is its drafter rank among its siblings; siblings carry distinct ranks;
    a rank with no listed probability has probability 0;
  * ridge tokens = peak dense flops x bytes per weight / (2 x HBM bandwidth) (two flops
    per weight per token); the tree size a batch B can afford is the largest N with
    B x N <= ridge, clamped to [1, max_nodes];
  * the best static tree of N nodes takes the N - 1 rank paths (length 1 .. max_depth)
    with the largest path products, ties going to the shorter, then the lexicographically
    smaller path; a path whose product is 0 is never taken.  The product of a path is
    formed root to leaf, one multiplication per step.
"""
import itertools
import math


def validate_ranked_tree(parent, rank):
    n = len(parent)
    if n < 1 or parent[0] != -1 or len(rank) != n:
        raise ValueError("bad tree")
    seen = set()
    for i in range(1, n):
        if not 0 <= parent[i] < i:
            raise ValueError("parent must precede child")
        if rank[i] < 0:
            raise ValueError("negative rank")
        key = (parent[i], rank[i])
        if key in seen:
            raise ValueError("siblings with equal ranks")
        seen.add(key)


def validate_probs(probs):
    if len(probs) < 1 or any(not (0.0 <= p <= 1.0) for p in probs) or sum(probs) > 1.0 + 1e-9:
        raise ValueError("rank probabilities must lie in [0, 1] and sum to at most 1")


def reach_probabilities(parent, rank, probs):
    """Probability that greedy verification reaches each node ([TAM] "What it buys"): the
    product of the rank probabilities along its path from the root; 1 at the root."""
    validate_ranked_tree(parent, rank)
    validate_probs(probs)
    out = []
    for i in range(len(parent)):
        path = []
        j = i
        while j > 0:
            path.append(rank[j])
            j = parent[j]
        p = 1.0
        for r in reversed(path):                     # root to leaf
            p *= probs[r] if r < len(probs) else 0.0
        out.append(p)
    return out


def expected_tokens(parent, rank, probs):
    """Expected tokens per step = 1 + the sum of the non-root nodes' reach probabilities
    ([TAM] "What it buys"; the root's 1 is the token the target always emits)."""
    reach = reach_probabilities(parent, rank, probs)
    return 1.0 + sum(reach[1:])


def ridge_tokens(peak_flops, hbm_bytes_per_s, bytes_per_weight):
    """Tokens per step at which a decode step stops being bandwidth-bound ([TAM] "What it
    costs": dense flops over bandwidth, for two-byte weights)."""
    return peak_flops * bytes_per_weight / (2.0 * hbm_bytes_per_s)


def nodes_for_batch(batch, ridge, max_nodes):
    """Largest N with batch x N <= ridge, within [1, max_nodes] ([TAM] "What it costs")."""
    if batch < 1 or max_nodes < 1 or not ridge >= 0:
        raise ValueError("bad budget arguments")
    return max(1, min(max_nodes, math.floor(ridge / batch)))


def path_product(path, probs):
    p = 1.0
    for r in path:
        p *= probs[r] if r < len(probs) else 0.0
    return p


def best_static_tree(probs, nodes, max_depth):
    """The N-node tree of most expected tokens ([TV] "The Cost Side"): every rank path up to
    max_depth is enumerated, ranked by (-product, length, path), and the first N - 1 with a
    non-zero product are kept.  Returns the paths in (length, lexicographic) order."""
    validate_probs(probs)
    if nodes < 1 or max_depth < 1:
        raise ValueError("bad budget arguments")
    cands = []
    for d in range(1, max_depth + 1):
        for path in itertools.product(range(len(probs)), repeat=d):
            p = path_product(path, probs)
            if p > 0.0:
                cands.append((-p, d, path))
    cands.sort()
    chosen = [c[2] for c in cands[:nodes - 1]]
    return sorted(chosen, key=lambda t: (len(t), t))


def plan(batch, ridge, probs, max_nodes, max_depth):
    """Tree size for the batch, then the best static tree of that size."""
    n = nodes_for_batch(batch, ridge, max_nodes)
    return n, best_static_tree(probs, n, max_depth)
