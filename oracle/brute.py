"""Per-node brute force: ordinary causal attention over each node's exact root path.
Test infrastructure (see ``oracle/__init__``).

The pages' correctness condition for tree verification is that node v's result equals
what a separate, ordinary causal pass over (cached prefix, root path of v) produces.
[TV, "Tree Attention" and "The Cost Side"; EBH: the recommended test checks a small
tree against one ordinary pass per node, on trees whose branches differ in length and
whose nodes reuse token labels]

So for every node i this module builds the ordinary sequence

    prefix positions 0..L-1, then the path root -> ... -> i at positions L, L+1, ..., L+d

and runs ``torch.nn.functional.scaled_dot_product_attention(is_causal=True,
enable_gqa=True)`` on it in float64 on the CPU -- a library routine that knows nothing
about trees, masks or bitmasks.  Its last row is node i's output.  The log-sum-exp comes
from ``scipy.special.logsumexp`` over the same sequence's scores.

An optional ``rope(x, positions)`` rotates queries and keys by their *sequential*
position in that ordinary sequence, which is the whole point of the rotary check: the
tree run must give node i position L + depth(i) for the two to agree.  [TAM, interviewer
probe on sibling positions and "Common mistakes"; EBH]
"""
import numpy as np
import torch
from scipy.special import logsumexp


def root_path(parent, i):
    """Nodes from the root down to ``i`` (inclusive), in path order."""
    up = []
    j = i
    guard = 0
    while j != -1:
        up.append(j)
        j = int(parent[j])
        guard += 1
        if guard > len(parent):
            raise ValueError("parent array has a cycle")
    return up[::-1]


def path_attention_request(q, k, v, parent, prefix_len, sm_scale=None, rope=None):
    """q: [N, Hq, D]; k, v: [>= L+N, Hkv, D] logical (prefix, then node j at L + j);
    returns out [N, Hq, D] and lse [N, Hq] (float64, natural log), node by node."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    L = int(prefix_len)
    scale = (1.0 / np.sqrt(d)) if sm_scale is None else float(sm_scale)
    out = np.zeros((n, hq, d))
    lse = np.zeros((n, hq))
    for i in range(n):
        path = root_path(parent, i)
        idx = list(range(L)) + [L + j for j in path]
        ks = k[idx]                                     # [T, Hkv, D], T = L + depth + 1
        vs = v[idx]
        T = len(idx)
        qs = np.zeros((T, hq, d))
        qs[L:] = q[path]                                # queries of the path's own nodes
        if rope is not None:
            seq_pos = np.arange(T)
            ks = rope(ks, seq_pos)
            qs = rope(qs, seq_pos)
        qt = torch.from_numpy(np.ascontiguousarray(qs.transpose(1, 0, 2)))[None]
        kt = torch.from_numpy(np.ascontiguousarray(ks.transpose(1, 0, 2)))[None]
        vt = torch.from_numpy(np.ascontiguousarray(vs.transpose(1, 0, 2)))[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, is_causal=True, scale=scale, enable_gqa=True)
        out[i] = o[0, :, T - 1, :].numpy()
        for h in range(hq):
            s = scale * (ks[:, h // g, :] @ qs[T - 1, h, :])
            lse[i, h] = logsumexp(s)
    return out, lse
