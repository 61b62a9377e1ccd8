"""Oracle: what happens after the verify pass -- TEST INFRASTRUCTURE ONLY.

Greedy acceptance on the tree and the compaction of the accepted path's KV entries, in
plain Python / numpy, sharing nothing with the HIP path.

Sources:
  [SV]  "Implement a batched speculative sampling verifier" (inferenceinterviews.com),
        "A strong answer" (the accept test u*q < p with no division, the residual
        max(0, p - q) a rejection is resampled from, the inverse-CDF draw and the p = q
        corner) and "What interviewers probe next" (a tree is walked from the root with
        the same rule, each sibling after a rejection judged against the residual).
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
  * stochastic walk: the children of a node are i.i.d. draws from that node's drafter
    distribution q (the case in which judging each sibling against the residual is
    exact); they are tested in node order; child c's test takes the uniform u[c] and the
    final draw (correction or bonus) takes u[0], the root never being tested; the
    arithmetic is float64;
  * inverse-CDF draw: the first index whose running sum exceeds u times the total (so an
    entry of weight zero is never drawn), the last entry of positive weight if rounding
    leaves none;
  * a rejection whose residual has no mass left (p = q within rounding, where the
    rejection had probability zero) leaves the distribution the next sibling is judged
    against unchanged, the tree form of the page's fall back to p.
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


def sample_inverse_cdf(weights, u):
    """One draw from non-negative ``weights`` (any positive total) by inverse CDF with the
    uniform ``u`` in [0, 1) ([SV] "A strong answer"): the first index whose running sum
    exceeds ``u`` times the total, or the last index of positive weight if none does."""
    w = np.asarray(weights, dtype=np.float64)
    if w.ndim != 1 or w.size == 0 or not np.all(np.isfinite(w)) or np.any(w < 0):
        raise ValueError("weights must be a non-empty vector of finite non-negative values")
    running = np.cumsum(w)
    total = running[-1]
    if not total > 0:
        raise ValueError("weights must have a positive total")
    past = np.flatnonzero(running > u * total)
    if past.size:
        return int(past[0])
    return int(np.flatnonzero(w > 0)[-1])


def _after_rejection(r, z, qn):
    """The distribution the next sibling is judged against after a rejection: the residual
    max(0, r / z - q), or r itself when the residual has no mass ([SV] "A strong answer":
    the residual and the p = q corner)."""
    residual = np.maximum(r / z - qn, 0.0)
    return residual if residual.sum() > 0 else r


def accept_stochastic(parent, draft, p, q, u):
    """Stochastic walk of the tree ([SV] "What interviewers probe next"; [TV] "Accepting
    on a Tree"), exact when every node's children are i.i.d. draws from its q.

    ``p[i]``: the target's next-token distribution after node i's path; ``q[i]``: the
    drafter's distribution at node i, from which node i's children were drawn;
    ``draft[c]``: child c's token; ``u[c]`` (c >= 1): the uniform of child c's test;
    ``u[0]``: the uniform of the final draw.  Distributions need not be normalised.

    Start at the root.  At the current node, r starts as its p.  Each child c in node
    order is tested: with z the total of r and x its token, c is accepted when
    u[c] * q(x) * z < r(x), i.e. with probability min(1, (r(x) / z) / q(x)) without
    dividing by q; the walk then emits x and moves to c.  After a rejection r becomes the
    residual max(0, r / z - q) (unchanged if that has no mass).  If no child is accepted
    (or the node is a leaf, where r is still p) one token is drawn from r with u[0] and
    the walk stops: a correction drawn from the residual, or the bonus token.

    Returns (accepted node indices, root first; emitted tokens), as accept_greedy.
    """
    parent = [int(x) for x in parent]
    _meta.validate_parent(parent)
    V = np.asarray(p[0]).shape[-1]
    if any(not 0 <= int(draft[c]) < V for c in range(1, len(parent))):
        raise ValueError("draft tokens must lie in [0, V)")
    table = child_table(parent)
    accepted, emitted = [0], []
    for _ in range(len(parent)):
        node = accepted[-1]
        r = np.asarray(p[node], dtype=np.float64).copy()
        qn = np.asarray(q[node], dtype=np.float64)
        taken = None
        for c in table[node]:
            x = int(draft[c])
            z = r.sum()
            if u[c] * qn[x] * z < r[x]:
                taken = c
                break
            r = _after_rejection(r, z, qn)
        if taken is None:
            emitted.append(sample_inverse_cdf(r, u[0]))
            break
        emitted.append(int(draft[taken]))
        accepted.append(taken)
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
