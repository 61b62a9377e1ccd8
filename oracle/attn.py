"""fp64 tree-verification attention, written as the plain masked-softmax definition.
Test infrastructure (see ``oracle/__init__``).

Definition followed:
* The full step mask of one request is the all-true block over the L cached prefix
  positions, beside the N x N tree mask; it has shape N x (L + N).  [TAM, "A strong
  answer", the paragraph after the build listing]
* Node i attends to every prefix position and to tree position L + j exactly when j is i
  or one of its ancestors; nothing else.  [TAM, "TL;DR"; TV, "Tree Attention"]
* Tree node j's key/value sits at logical position L + j, in node order.  [TAM, "What it
  costs": the tree's cache rows sit in node order]
* Under that mask one pass gives every node the same result a separate causal pass over
  its own root path would give.  [TV, "Tree Attention"; EBH]

Conventions the pages leave open (shared with the HIP path only as written spec):
* grouped-query attention: query head h reads kv head ``h // (Hq // Hkv)``;
* scores are ``sm_scale * <q, k>`` with ``sm_scale = 1/sqrt(D)`` unless given;
* ``lse`` is the natural-log log-sum-exp of the allowed scores;
* inputs are upcast to float64 from exactly the values the device sees (bf16 bit
  patterns are decoded here by this module's own decoder).

No blocking, splitting or online rescaling: one dense masked softmax per (request, head).
"""
import numpy as np

from . import meta as _meta


def bf16_bits_to_f64(bits):
    """Decode bfloat16 bit patterns (uint16 array) to float64.  A bfloat16 value is the
    upper half of an IEEE-754 binary32, so the binary32 pattern is ``bits << 16``."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def gather_paged(pool, page_table_row, page_size, length):
    """Logical K or V of one request from a paged pool.

    ``pool``: [num_pages, page_size, Hkv, D]; logical token t lives in physical page
    ``page_table_row[t // page_size]`` at slot ``t % page_size``.  Returns [length, Hkv, D].
    """
    pool = np.asarray(pool)
    rows = []
    for t in range(length):
        rows.append(pool[int(page_table_row[t // page_size]), t % page_size])
    if not rows:
        return pool[:0, 0]
    return np.stack(rows, axis=0)


def step_mask(parent, prefix_len):
    """The full step mask [N, L + N] (bool): all prefix columns true, then the tree mask."""
    tree = np.array(_meta.dense_mask(list(parent)), dtype=bool)
    n = tree.shape[0]
    return np.concatenate([np.ones((n, prefix_len), dtype=bool), tree], axis=1)


def tree_attention_request(q, k, v, parent, prefix_len, sm_scale=None, kv_heads=None):
    """Tree attention for one request.

    q: [N, Hq, D]; k, v: [>= L + N, Hkv, D] in logical token order (prefix then tree nodes
    in node order); parent: [N] parent-before-child; prefix_len: L.
    ``kv_heads``: optional subset of kv heads to evaluate (others are left NaN).
    Returns ``out`` [N, Hq, D] float64 and ``lse`` [N, Hq] float64 (natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    parent = [int(x) for x in parent]
    _meta.validate_parent(parent)
    n, hq, d = q.shape
    hkv = k.shape[1]
    if len(parent) != n:
        raise ValueError("parent length must equal the number of tree nodes")
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    L = int(prefix_len)
    total = L + n
    if k.shape[0] < total or v.shape[0] < total:
        raise ValueError("k/v must hold the prefix and every tree node")
    scale = (1.0 / np.sqrt(d)) if sm_scale is None else float(sm_scale)
    allowed = step_mask(parent, L)                       # [N, L+N]
    out = np.full((n, hq, d), np.nan)
    lse = np.full((n, hq), np.nan)
    heads = range(hkv) if kv_heads is None else kv_heads
    for kh in heads:
        keys = k[:total, kh, :]                          # [L+N, D]
        vals = v[:total, kh, :]
        for j in range(g):
            h = kh * g + j
            s = scale * (q[:, h, :] @ keys.T)            # [N, L+N]
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            out[:, h, :] = (e / z) @ vals
            lse[:, h] = (m + np.log(z))[:, 0]
    return out, lse


def tree_attention(q, k, v, parent, prefix_len, sm_scale=None):
    """Batched form over contiguous logical K/V.

    q: [B, N, Hq, D]; k, v: [B, S, Hkv, D] with S >= max(prefix_len) + N (logical order);
    parent: [B, N] (or [N], one tree shared by every request); prefix_len: [B].
    Returns out [B, N, Hq, D], lse [B, N, Hq] (float64, natural log).
    """
    q = np.asarray(q)
    B = q.shape[0]
    parent = np.asarray(parent)
    outs, lses = [], []
    for b in range(B):
        pb = parent if parent.ndim == 1 else parent[b]
        o, l = tree_attention_request(q[b], k[b], v[b], pb, int(prefix_len[b]), sm_scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
