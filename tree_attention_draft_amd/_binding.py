"""ctypes binding of libtreeverify.so (see include/tree_verify.h).

Marshalling only: every step of the path runs in the library's HIP kernels or its host C++
builder.  PyTorch supplies device memory and the current stream.  If the shared library
is missing this module raises on first use -- there is no fallback.
"""
import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtreeverify.so")

TV_OK = 0
STATUS_NAMES = {0: "TV_OK", 1: "TV_ERR_INVALID_ARG", 2: "TV_ERR_INVALID_PATH",
                3: "TV_ERR_MISSING_PARENT", 4: "TV_ERR_CAPACITY", 5: "TV_ERR_UNSUPPORTED",
                6: "TV_ERR_WORKSPACE", 7: "TV_ERR_HIP"}
TV_BF16, TV_F32 = 0, 1
TV_KV_CONTIGUOUS, TV_KV_PAGED = 0, 1
PATHS = {"auto": 0, "valu": 1, "mfma": 2}
MAX_NODES = 64

# Every symbol include/tree_verify.h declares.
EXPORTS = ["tree_meta_build", "tree_meta_build_batch", "tree_meta_from_parent",
           "tree_verify_attn_workspace_size", "tree_verify_attn", "tree_verify_attn_static",
           "tree_accept_greedy",
           "tree_accept_greedy_workspace_size", "tree_accept_stochastic",
           "tree_kv_compact", "tree_expected_tokens", "tree_ridge_tokens",
           "tree_budget_nodes", "tree_best_static", "tree_budget_plan",
           "tv_status_string", "tv_last_error", "tv_abi_version", "tv_pinned_device_address",
           "tv_attn_args_sizeof", "tv_accept_args_sizeof", "tv_sample_args_sizeof",
           "tv_compact_args_sizeof"]


class TreeVerifyError(RuntimeError):
    def __init__(self, status, detail, bad_path=-1, bad_tree=-1):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        self.bad_path = bad_path
        self.bad_tree = bad_tree
        super().__init__(f"{self.name}: {detail}" + (
            f" (input path {bad_path})" if bad_path >= 0 else ""))


class TvAttnArgs(ctypes.Structure):
    """Mirror of ``tv_attn_args`` (field order and types must match the header)."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("N", ctypes.c_int32),
        ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_sb", ctypes.c_int64), ("q_sn", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("kv_layout", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_sb", ctypes.c_int64), ("kv_st", ctypes.c_int64), ("kv_sh", ctypes.c_int64),
        ("page_table", ctypes.c_void_p),
        ("pages_per_seq", ctypes.c_int32), ("parent_sb", ctypes.c_int32),
        ("parent", ctypes.c_void_p), ("prefix_len", ctypes.c_void_p),
        ("max_prefix_len", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("o_sb", ctypes.c_int64), ("o_sn", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("num_splits", ctypes.c_int32), ("path", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("prefix_len_host", ctypes.c_void_p),
        ("meta_depth", ctypes.c_void_p), ("meta_bitmask", ctypes.c_void_p),
        ("meta_pos", ctypes.c_void_p),
    ]


class TvAcceptArgs(ctypes.Structure):
    """Mirror of ``tv_accept_args``."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("N", ctypes.c_int32),
        ("V", ctypes.c_int32), ("logits", ctypes.c_void_p),
        ("lg_sb", ctypes.c_int64), ("lg_sn", ctypes.c_int64),
        ("tokens", ctypes.c_void_p), ("tokens_sb", ctypes.c_int32),
        ("parent", ctypes.c_void_p), ("parent_sb", ctypes.c_int32),
        ("target", ctypes.c_void_p), ("accepted", ctypes.c_void_p),
        ("emitted", ctypes.c_void_p), ("num_accepted", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class TvSampleArgs(ctypes.Structure):
    """Mirror of ``tv_sample_args``."""
    _fields_ = [
        ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("V", ctypes.c_int32),
        ("p", ctypes.c_void_p), ("p_sb", ctypes.c_int64), ("p_sn", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_sn", ctypes.c_int64),
        ("tokens", ctypes.c_void_p), ("tokens_sb", ctypes.c_int32),
        ("parent", ctypes.c_void_p), ("parent_sb", ctypes.c_int32),
        ("uniform", ctypes.c_void_p), ("uniform_sb", ctypes.c_int32),
        ("accepted", ctypes.c_void_p), ("emitted", ctypes.c_void_p),
        ("num_accepted", ctypes.c_void_p),
    ]


class TvCompactArgs(ctypes.Structure):
    """Mirror of ``tv_compact_args``."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("N", ctypes.c_int32),
        ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("kv_layout", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_sb", ctypes.c_int64), ("kv_st", ctypes.c_int64), ("kv_sh", ctypes.c_int64),
        ("page_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32),
        ("prefix_len", ctypes.c_void_p), ("max_prefix_len", ctypes.c_int32),
        ("parent", ctypes.c_void_p), ("parent_sb", ctypes.c_int32),
        ("accepted", ctypes.c_void_p), ("num_accepted", ctypes.c_void_p),
        ("new_len", ctypes.c_void_p), ("status", ctypes.c_void_p),
        ("rope_theta", ctypes.c_double),
    ]


_LIB = None


def lib():
    """The loaded library (loads it on first call; raises if it was never built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m tree_attention_draft_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.tree_meta_build.restype = i32
    L.tree_meta_build.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.tree_meta_build_batch.restype = i32
    L.tree_meta_build_batch.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    L.tree_meta_from_parent.restype = i32
    L.tree_meta_from_parent.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
    L.tree_verify_attn_workspace_size.restype = ctypes.c_size_t
    L.tree_verify_attn_workspace_size.argtypes = [ctypes.POINTER(TvAttnArgs)]
    L.tree_verify_attn.restype = i32
    L.tree_verify_attn.argtypes = [ctypes.POINTER(TvAttnArgs), vp]
    L.tree_verify_attn_static.restype = i32
    L.tree_verify_attn_static.argtypes = [ctypes.POINTER(TvAttnArgs), vp]
    L.tv_status_string.restype = ctypes.c_char_p
    L.tv_status_string.argtypes = [i32]
    L.tv_last_error.restype = ctypes.c_char_p
    L.tv_last_error.argtypes = []
    L.tv_abi_version.restype = i32
    L.tv_pinned_device_address.restype = i32
    L.tv_pinned_device_address.argtypes = [vp, ctypes.POINTER(vp)]
    L.tv_attn_args_sizeof.restype = ctypes.c_size_t
    L.tree_accept_greedy_workspace_size.restype = ctypes.c_size_t
    L.tree_accept_greedy_workspace_size.argtypes = [ctypes.POINTER(TvAcceptArgs)]
    L.tree_accept_greedy.restype = i32
    L.tree_accept_greedy.argtypes = [ctypes.POINTER(TvAcceptArgs), vp]
    L.tree_accept_stochastic.restype = i32
    L.tree_accept_stochastic.argtypes = [ctypes.POINTER(TvSampleArgs), vp]
    L.tv_sample_args_sizeof.restype = ctypes.c_size_t
    L.tree_kv_compact.restype = i32
    L.tree_kv_compact.argtypes = [ctypes.POINTER(TvCompactArgs), vp]
    L.tv_accept_args_sizeof.restype = ctypes.c_size_t
    L.tv_compact_args_sizeof.restype = ctypes.c_size_t
    f64, i64 = ctypes.c_double, ctypes.c_int64
    L.tree_expected_tokens.restype = i32
    L.tree_expected_tokens.argtypes = [vp, vp, i32, vp, i32, vp, vp]
    L.tree_ridge_tokens.restype = i32
    L.tree_ridge_tokens.argtypes = [f64, f64, f64, vp]
    L.tree_budget_nodes.restype = i32
    L.tree_budget_nodes.argtypes = [i32, f64, i32, vp]
    L.tree_best_static.restype = i32
    L.tree_best_static.argtypes = [vp, i32, i32, i32, vp, i64, vp, vp, vp]
    L.tree_budget_plan.restype = i32
    L.tree_budget_plan.argtypes = [i32, f64, i32, vp, i32, i32, vp, vp, i64, vp, vp, vp]
    _LIB = L
    return L


def _check(status, bad_path=-1):
    if status != TV_OK:
        raise TreeVerifyError(status, lib().tv_last_error().decode(), bad_path)


# ------------------------------------------------------------------- host builder ----
def tree_meta_build(paths, prefix_len, max_nodes=MAX_NODES):
    """Rank paths -> dict of numpy arrays ``parent``, ``depth``, ``bitmask`` (uint64),
    ``pos`` (length N), built by the library's host C++ builder."""
    offs = [0]
    flat = []
    for p in paths:
        flat.extend(int(x) for x in p)
        offs.append(len(flat))
    ranks = np.asarray(flat if flat else [0], dtype=np.int32)
    path_off = np.asarray(offs, dtype=np.int64)
    cap = int(max_nodes)
    parent = np.empty(cap, np.int32)
    depth = np.empty(cap, np.int32)
    bitmask = np.empty(cap, np.uint64)
    pos = np.empty(cap, np.int32)
    n = ctypes.c_int32(0)
    bad = ctypes.c_int32(-1)
    st = lib().tree_meta_build(
        ranks.ctypes.data, path_off.ctypes.data, len(paths), int(prefix_len), cap,
        parent.ctypes.data, depth.ctypes.data, bitmask.ctypes.data, pos.ctypes.data,
        ctypes.byref(n), ctypes.byref(bad))
    _check(st, bad.value)
    k = n.value
    return {"parent": parent[:k].copy(), "depth": depth[:k].copy(),
            "bitmask": bitmask[:k].copy(), "pos": pos[:k].copy()}


class PackedTrees:
    """Candidate paths of B requests packed once as CSR arrays (host memory), ready for
    repeated tree_meta_build_batch calls."""

    def __init__(self, trees):
        offs, flat, toff = [0], [], [0]
        for paths in trees:
            for p in paths:
                flat.extend(int(x) for x in p)
                offs.append(len(flat))
            toff.append(len(offs) - 1)
        self.ranks = np.asarray(flat if flat else [0], dtype=np.int32)
        self.path_off = np.asarray(offs, dtype=np.int64)
        self.tree_off = np.asarray(toff, dtype=np.int64)
        self.B = len(trees)


def tree_meta_build_batch(packed, prefix_len, N, parent=None, depth=None, bitmask=None,
                          pos=None):
    """Build all B trees of ``packed`` (a :class:`PackedTrees`) into dense [B, N] host
    arrays.  Output arrays may be passed in (e.g. pinned buffers viewed as numpy)."""
    B = packed.B
    pl = np.ascontiguousarray(prefix_len, dtype=np.int32)
    parent = np.empty((B, N), np.int32) if parent is None else parent
    depth = np.empty((B, N), np.int32) if depth is None else depth
    bitmask = np.empty((B, N), np.uint64) if bitmask is None else bitmask
    pos = np.empty((B, N), np.int32) if pos is None else pos
    nn = np.empty(B, np.int32)
    bt, bp = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = lib().tree_meta_build_batch(
        packed.ranks.ctypes.data, packed.path_off.ctypes.data, packed.tree_off.ctypes.data,
        B, pl.ctypes.data, int(N), parent.ctypes.data, depth.ctypes.data,
        bitmask.ctypes.data, pos.ctypes.data, nn.ctypes.data, ctypes.byref(bt),
        ctypes.byref(bp))
    if st != TV_OK:
        raise TreeVerifyError(st, lib().tv_last_error().decode() + f" (tree {bt.value})",
                              bp.value, bt.value)
    return {"parent": parent, "depth": depth, "bitmask": bitmask, "pos": pos,
            "num_nodes": nn}


class PreparedBuild:
    """A ``tree_meta_build_batch`` call with every pointer resolved once: calling it only
    runs the C builder into the same output arrays (a serving loop's per-step metadata).
    Keeps the packed trees, prefix lengths and outputs alive; their contents may change
    between calls, their storage may not.  Prefix lengths given as a C-contiguous int32
    array are read in place (otherwise from a copy made here)."""

    def __init__(self, packed, prefix_len, N, parent, depth, bitmask, pos):
        self._keep = (packed, np.ascontiguousarray(prefix_len, dtype=np.int32), parent,
                      depth, bitmask, pos, np.empty(packed.B, np.int32))
        pl, nn = self._keep[1], self._keep[6]
        for a, dt in ((parent, np.int32), (depth, np.int32), (bitmask, np.uint64),
                      (pos, np.int32)):
            if a.dtype != dt or a.shape != (packed.B, N) or not a.flags.c_contiguous:
                raise ValueError("outputs must be C-contiguous [B, N] int32/int32/uint64/int32")
        self._bt, self._bp = ctypes.c_int32(-1), ctypes.c_int32(-1)
        self._args = (packed.ranks.ctypes.data, packed.path_off.ctypes.data,
                      packed.tree_off.ctypes.data, packed.B, pl.ctypes.data, int(N),
                      parent.ctypes.data, depth.ctypes.data, bitmask.ctypes.data,
                      pos.ctypes.data, nn.ctypes.data, ctypes.byref(self._bt),
                      ctypes.byref(self._bp))
        self.num_nodes = nn

    def __call__(self):
        st = lib().tree_meta_build_batch(*self._args)
        if st != TV_OK:
            raise TreeVerifyError(st, lib().tv_last_error().decode() +
                                  f" (tree {self._bt.value})", self._bp.value, self._bt.value)


def prepare_tree_meta_build_batch(packed, prefix_len, N, parent, depth, bitmask, pos):
    """``tree_meta_build_batch`` into the given [B, N] host arrays (numpy, e.g. views of
    pinned buffers), prepared once: returns a :class:`PreparedBuild`."""
    return PreparedBuild(packed, prefix_len, N, parent, depth, bitmask, pos)


# ------------------------------------------------------------------- device side -----
def _torch():
    import torch
    return torch


def _torch_stream(stream):
    """The torch stream the kernels are enqueued on: ``stream``, else the current one."""
    torch = _torch()
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


def _on(stream):
    """Context in which buffers this module creates are allocated on the launch stream.
    The caching allocator then hands such a buffer to other work only in that stream's
    order, i.e. after the kernels that write it -- also for the split workspace, which is
    dropped when the call returns while its kernels may still be running."""
    return _torch().cuda.stream(_torch_stream(stream))


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("tree-verify device entry points take GPU tensors")


def _parent_address(parent):
    """Address the kernels read ``parent`` at: a GPU tensor's own, or the device address of
    a pinned host tensor (the pass reads it in place, so the host may refill such a buffer
    only after the pass that reads it has finished)."""
    if parent.is_cuda:
        return parent.data_ptr()
    if not parent.is_pinned():
        raise ValueError("parent must be a GPU tensor or a pinned host tensor")
    dev = ctypes.c_void_p()
    _check(lib().tv_pinned_device_address(ctypes.c_void_p(parent.data_ptr()), ctypes.byref(dev)))
    return dev.value


def tree_meta_from_parent(parent, prefix_len=None, batch=None, depth=None, bitmask=None,
                          pos=None, stream=None):
    """Device metadata from int32 parent arrays ``[B, N]`` (or ``[N]`` shared by ``batch``
    requests).  Returns ``(depth, bitmask, pos)`` as [B, N] tensors (int32, int64 holding
    the uint64 bit pattern, int32)."""
    torch = _torch()
    _require_cuda(parent, prefix_len)
    if parent.dtype != torch.int32:
        raise ValueError("parent must be int32")
    if parent.dim() == 1:
        if batch is None:
            batch = prefix_len.shape[0] if prefix_len is not None else 1
        B, N, psb = int(batch), parent.shape[0], 0
    else:
        B, N = parent.shape
        psb = parent.stride(0)
        if parent.stride(1) != 1:
            raise ValueError("parent rows must be contiguous")
    dev = parent.device
    with _on(stream):
        depth = torch.empty((B, N), dtype=torch.int32, device=dev) if depth is None else depth
        bitmask = (torch.empty((B, N), dtype=torch.int64, device=dev) if bitmask is None
                   else bitmask)
        pos = torch.empty((B, N), dtype=torch.int32, device=dev) if pos is None else pos
    st = lib().tree_meta_from_parent(
        parent.data_ptr(), psb, B, N,
        prefix_len.data_ptr() if prefix_len is not None else None,
        depth.data_ptr(), bitmask.data_ptr(), pos.data_ptr(), _stream(stream))
    _check(st)
    return depth, bitmask, pos


def make_args(q, k, v, parent, prefix_len, max_prefix_len, page_table=None, page_size=0,
              sm_scale=0.0, out=None, lse=None, workspace=None, num_splits=0, path="auto",
              rope_theta=0.0, prefix_len_host=None, meta=None):
    """Fill a TvAttnArgs from torch tensors (no allocation, no checks beyond shapes).
    ``prefix_len_host``: optional host copy of the prefix lengths (int32 numpy array of B
    values) for the split plan; the returned struct keeps it alive.  ``parent`` may be a
    pinned host tensor (read in place).  ``meta``: optional (depth, bitmask, pos) [B, N]
    GPU tensors (int32, int64, int32; any may be None) the pass also fills."""
    torch = _torch()
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    a = TvAttnArgs()
    if q.dtype == torch.bfloat16:
        a.dtype = TV_BF16
    elif q.dtype == torch.float32:
        a.dtype = TV_F32
    else:
        raise ValueError("q must be bfloat16 or float32")
    a.B, a.N, a.Hq, a.Hkv, a.D = B, N, Hq, Hkv, D
    a.q = q.data_ptr()
    a.q_sb, a.q_sn, a.q_sh = q.stride(0), q.stride(1), q.stride(2)
    a.k, a.v = k.data_ptr(), v.data_ptr()
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    a.kv_sb, a.kv_st, a.kv_sh = k.stride(0), k.stride(1), k.stride(2)
    if page_table is not None:
        a.kv_layout = TV_KV_PAGED
        a.page_size = int(page_size) if page_size else k.shape[1]
        a.page_table = page_table.data_ptr()
        a.pages_per_seq = page_table.shape[1]
    else:
        a.kv_layout = TV_KV_CONTIGUOUS
    if parent.dim() == 1:
        a.parent_sb = 0
    else:
        a.parent_sb = parent.stride(0)
    a.parent = _parent_address(parent)
    a.prefix_len = prefix_len.data_ptr()
    a.max_prefix_len = int(max_prefix_len)
    a.sm_scale = float(sm_scale)
    if out is not None:
        a.out = out.data_ptr()
        a.o_sb, a.o_sn, a.o_sh = out.stride(0), out.stride(1), out.stride(2)
    a.lse = lse.data_ptr() if lse is not None else None
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.num_splits = int(num_splits)
    a.path = PATHS[path] if isinstance(path, str) else int(path)
    a.rope_theta = float(rope_theta)
    if prefix_len_host is not None:
        hint = np.ascontiguousarray(prefix_len_host, dtype=np.int32)
        if hint.shape != (B,):
            raise ValueError("prefix_len_host must hold B values")
        a._hint = hint
        a.prefix_len_host = hint.ctypes.data
    if meta is not None:
        depth, bitmask, pos = meta
        a.meta_depth = depth.data_ptr() if depth is not None else None
        a.meta_bitmask = bitmask.data_ptr() if bitmask is not None else None
        a.meta_pos = pos.data_ptr() if pos is not None else None
    return a


def tree_verify_attn_workspace_size(q, k, v, parent, prefix_len, max_prefix_len, **kw):
    a = make_args(q, k, v, parent, prefix_len, max_prefix_len, **kw)
    return int(lib().tree_verify_attn_workspace_size(ctypes.byref(a)))


def tree_verify_attn(q, k, v, parent, prefix_len, max_prefix_len, *, page_table=None,
                     page_size=0, sm_scale=0.0, out=None, lse=None, workspace=None,
                     num_splits=0, path="auto", rope_theta=0.0, prefix_len_host=None,
                     meta=None, stream=None):
    """Tree-verification attention.  q [B, N, Hq, D]; k, v [B, S, Hkv, D] (contiguous) or
    [pages, page_size, Hkv, D] with ``page_table`` [B, pages_per_seq]; parent int32 [B, N]
    or [N] (a GPU tensor, or a pinned host tensor read in place); prefix_len int32 [B].
    ``rope_theta`` > 0 fuses the rotary embedding: q and the tree keys are passed
    unrotated and rotated at L + depth inside the kernels.  ``meta``: optional
    (depth, bitmask, pos) [B, N] GPU tensors that also receive the expanded tree, as
    ``tree_meta_from_parent`` writes it.  Returns ``(out, lse)``; ``lse`` is the
    natural-log log-sum-exp per (request, node, query head)."""
    torch = _torch()
    _require_cuda(q, k, v, prefix_len, page_table, out, lse, workspace)
    if meta is not None:
        _require_cuda(*meta)
        for t, dt in zip(meta, (torch.int32, torch.int64, torch.int32)):
            if t is not None and (t.dtype != dt or t.numel() != _dense_bn(q)
                                  or not t.is_contiguous()):
                raise ValueError("meta outputs must be contiguous [B, N] int32/int64/int32")
    B, N, Hq, D = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, N, Hq), dtype=torch.float32, device=q.device)
    a = make_args(q, k, v, parent, prefix_len, max_prefix_len, page_table=page_table,
                  page_size=page_size, sm_scale=sm_scale, out=out, lse=lse,
                  workspace=workspace, num_splits=num_splits, path=path,
                  rope_theta=rope_theta, prefix_len_host=prefix_len_host, meta=meta)
    need = int(lib().tree_verify_attn_workspace_size(ctypes.byref(a)))
    if need > 0 and (workspace is None or a.workspace_bytes < need):
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = need
    st = lib().tree_verify_attn(ctypes.byref(a), _stream(stream))
    _check(st)
    return out, lse


class PreparedAttn:
    """A ``tree_verify_attn`` call whose arguments are marshalled once: calling it only
    enqueues the pass (the C call with the prepared struct), so a serving loop that reuses
    the same buffers pays no per-call argument handling.  It keeps the tensors it was made
    from alive; their contents may change between calls, their storage may not.  Calls on
    one object share its output and workspace buffers: the caller orders them."""

    def __init__(self, args, keep, stream):
        self._a = args
        self._ref = ctypes.byref(args)
        self._fn = lib().tree_verify_attn
        self._keep = keep
        self._stream = stream
        self.out, self.lse = keep["out"], keep["lse"]

    def __call__(self):
        _check(self._fn(self._ref, self._stream))
        return self.out, self.lse


def prepare_tree_verify_attn(q, k, v, parent, prefix_len, max_prefix_len, *, out,
                             lse=None, workspace=None, page_table=None, page_size=0,
                             sm_scale=0.0, num_splits=0, path="auto", rope_theta=0.0,
                             prefix_len_host=None, meta=None, stream=None):
    """Marshal the arguments of ``tree_verify_attn`` once (same meaning) and return a
    :class:`PreparedAttn` that launches the pass on ``stream`` each time it is called
    (when None, on the stream that is current now, at preparation, not at each call).
    ``out`` is required; the split workspace is taken from ``workspace`` when it is large
    enough, else allocated here once on that stream."""
    torch = _torch()
    _require_cuda(q, k, v, prefix_len, page_table, out, lse, workspace)
    a = make_args(q, k, v, parent, prefix_len, max_prefix_len, page_table=page_table,
                  page_size=page_size, sm_scale=sm_scale, out=out, lse=lse,
                  workspace=workspace, num_splits=num_splits, path=path,
                  rope_theta=rope_theta, prefix_len_host=prefix_len_host, meta=meta)
    need = int(lib().tree_verify_attn_workspace_size(ctypes.byref(a)))
    if need > 0 and (workspace is None or a.workspace_bytes < need):
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = need
    keep = dict(q=q, k=k, v=v, parent=parent, prefix_len=prefix_len, page_table=page_table,
                out=out, lse=lse, workspace=workspace, meta=meta)
    return PreparedAttn(a, keep, _stream(stream))


STATIC_SCRATCH_BYTES = 64 * 1024 * 1024   # TV_STATIC_SCRATCH_BYTES


def tree_verify_attn_static(q, k, v, parent, prefix_len, max_prefix_len, *, out, lse=None,
                            page_table=None, page_size=0, sm_scale=0.0, num_splits=0,
                            path="auto", rope_theta=0.0, prefix_len_host=None, meta=None,
                            stream=None):
    """``tree_verify_attn`` without any device allocation: the caller passes ``out`` (and
    ``lse`` if wanted); the split workspace is the library's static device array.
    Raises TreeVerifyError (TV_ERR_WORKSPACE) when the plan needs more than
    ``STATIC_SCRATCH_BYTES`` of workspace."""
    _require_cuda(q, k, v, prefix_len, page_table, out, lse)
    a = make_args(q, k, v, parent, prefix_len, max_prefix_len, page_table=page_table,
                  page_size=page_size, sm_scale=sm_scale, out=out, lse=lse,
                  num_splits=num_splits, path=path, rope_theta=rope_theta,
                  prefix_len_host=prefix_len_host, meta=meta)
    _check(lib().tree_verify_attn_static(ctypes.byref(a), _stream(stream)))
    return out, lse


def _dense_bn(q):
    """Elements of a dense [B, N] array for queries ``q`` [B, N, Hq, D]."""
    return q.shape[0] * q.shape[1]


def default_scale(D):
    return 1.0 / math.sqrt(D)


# ------------------------------------------------------------ after the pass --------
def _rows(t, name, B, N, dtype=None):
    """Request stride of an int32 (or ``dtype``) [B, N] (or shared [N]) tensor."""
    torch = _torch()
    dtype = torch.int32 if dtype is None else dtype
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if t.dim() == 1:
        if t.shape[0] != N:
            raise ValueError(f"{name} must have N entries")
        return 0
    if tuple(t.shape) != (B, N) or t.stride(1) != 1:
        raise ValueError(f"{name} must be [B, N] with contiguous rows")
    return t.stride(0)


def make_accept_args(logits, tokens, parent, target, accepted, emitted, num_accepted):
    torch = _torch()
    B, N, V = logits.shape
    a = TvAcceptArgs()
    if logits.dtype == torch.bfloat16:
        a.dtype = TV_BF16
    elif logits.dtype == torch.float32:
        a.dtype = TV_F32
    else:
        raise ValueError("logits must be bfloat16 or float32")
    if logits.stride(2) != 1:
        raise ValueError("logits must be contiguous along the vocabulary")
    a.B, a.N, a.V = B, N, V
    a.logits = logits.data_ptr()
    a.lg_sb, a.lg_sn = logits.stride(0), logits.stride(1)
    a.tokens_sb = _rows(tokens, "tokens", B, N)
    a.tokens = tokens.data_ptr()
    a.parent_sb = _rows(parent, "parent", B, N)
    a.parent = parent.data_ptr()
    for t, n in ((target, "target"), (accepted, "accepted"), (emitted, "emitted")):
        if t.dtype != torch.int32 or tuple(t.shape) != (B, N) or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 [B, N] tensor")
    if num_accepted.dtype != torch.int32 or tuple(num_accepted.shape) != (B,):
        raise ValueError("num_accepted must be int32 [B]")
    a.target, a.accepted = target.data_ptr(), accepted.data_ptr()
    a.emitted, a.num_accepted = emitted.data_ptr(), num_accepted.data_ptr()
    return a


def tree_accept_greedy(logits, tokens, parent, target=None, accepted=None, emitted=None,
                       num_accepted=None, workspace=None, stream=None):
    """Greedy verification: ``logits`` [B, N, V] (bf16 or fp32), draft ``tokens`` and
    ``parent`` int32 [B, N] (or [N] shared).  Returns ``(target, accepted, emitted,
    num_accepted)``: the target's greedy token per node, the accepted nodes (root first,
    -1 padded), the emitted tokens (-1 padded) and their count per request."""
    torch = _torch()
    _require_cuda(logits, tokens, parent, target, accepted, emitted, num_accepted)
    B, N, _ = logits.shape
    dev = logits.device
    def mk(t, shape):
        return torch.empty(shape, dtype=torch.int32, device=dev) if t is None else t
    with _on(stream):
        target, accepted = mk(target, (B, N)), mk(accepted, (B, N))
        emitted, num_accepted = mk(emitted, (B, N)), mk(num_accepted, (B,))
    a = make_accept_args(logits, tokens, parent, target, accepted, emitted, num_accepted)
    need = int(lib().tree_accept_greedy_workspace_size(ctypes.byref(a)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        with _on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tree_accept_greedy(ctypes.byref(a), _stream(stream)))
    return target, accepted, emitted, num_accepted


def make_sample_args(p, q, tokens, parent, uniform, accepted, emitted, num_accepted):
    torch = _torch()
    if p.dim() != 3 or q.shape != p.shape:
        raise ValueError("p and q must be [B, N, V] of the same shape")
    for t, n in ((p, "p"), (q, "q")):
        if t.dtype != torch.float32 or t.stride(2) != 1:
            raise ValueError(f"{n} must be float32, contiguous along the vocabulary")
    B, N, V = p.shape
    a = TvSampleArgs()
    a.B, a.N, a.V = B, N, V
    a.p, a.p_sb, a.p_sn = p.data_ptr(), p.stride(0), p.stride(1)
    a.q, a.q_sb, a.q_sn = q.data_ptr(), q.stride(0), q.stride(1)
    a.tokens_sb = _rows(tokens, "tokens", B, N)
    a.tokens = tokens.data_ptr()
    a.parent_sb = _rows(parent, "parent", B, N)
    a.parent = parent.data_ptr()
    a.uniform_sb = _rows(uniform, "uniform", B, N, torch.float64)
    a.uniform = uniform.data_ptr()
    for t, n in ((accepted, "accepted"), (emitted, "emitted")):
        if t.dtype != torch.int32 or tuple(t.shape) != (B, N) or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 [B, N] tensor")
    if num_accepted.dtype != torch.int32 or tuple(num_accepted.shape) != (B,):
        raise ValueError("num_accepted must be int32 [B]")
    a.accepted, a.emitted = accepted.data_ptr(), emitted.data_ptr()
    a.num_accepted = num_accepted.data_ptr()
    return a


def tree_accept_stochastic(p, q, tokens, parent, uniform, accepted=None, emitted=None,
                           num_accepted=None, stream=None):
    """Stochastic verification: target ``p`` and drafter ``q`` distributions [B, N, V]
    (float32), draft ``tokens``, ``parent`` int32 and ``uniform`` float64 in [0, 1), each
    [B, N] (or [N] shared).  Returns ``(accepted, emitted, num_accepted)`` as
    tree_accept_greedy does."""
    torch = _torch()
    _require_cuda(p, q, tokens, parent, uniform, accepted, emitted, num_accepted)
    B, N, _ = p.shape
    dev = p.device
    def mk(t, shape):
        return torch.empty(shape, dtype=torch.int32, device=dev) if t is None else t
    with _on(stream):
        accepted, emitted = mk(accepted, (B, N)), mk(emitted, (B, N))
        num_accepted = mk(num_accepted, (B,))
    a = make_sample_args(p, q, tokens, parent, uniform, accepted, emitted, num_accepted)
    _check(lib().tree_accept_stochastic(ctypes.byref(a), _stream(stream)))
    return accepted, emitted, num_accepted


def make_compact_args(k, v, prefix_len, max_prefix_len, parent, accepted, num_accepted,
                      page_table=None, page_size=0, new_len=None, status=None,
                      rope_theta=0.0):
    torch = _torch()
    a = TvCompactArgs()
    a.rope_theta = float(rope_theta)
    if k.dtype == torch.bfloat16:
        a.dtype = TV_BF16
    elif k.dtype == torch.float32:
        a.dtype = TV_F32
    else:
        raise ValueError("k must be bfloat16 or float32")
    if k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must share dtype and strides")
    B = prefix_len.shape[0]
    N = accepted.shape[1]
    a.B, a.N, a.Hkv, a.D = B, N, k.shape[2], k.shape[3]
    a.k, a.v = k.data_ptr(), v.data_ptr()
    a.kv_sb, a.kv_st, a.kv_sh = k.stride(0), k.stride(1), k.stride(2)
    if page_table is not None:
        a.kv_layout = TV_KV_PAGED
        a.page_table = page_table.data_ptr()
        a.page_size = int(page_size) if page_size else k.shape[1]
        a.pages_per_seq = page_table.shape[1]
    else:
        a.kv_layout = TV_KV_CONTIGUOUS
    a.prefix_len = prefix_len.data_ptr()
    a.max_prefix_len = int(max_prefix_len)
    a.parent_sb = _rows(parent, "parent", B, N)
    a.parent = parent.data_ptr()
    if _rows(accepted, "accepted", B, N) != N:
        raise ValueError("accepted must be a contiguous [B, N] tensor")
    a.accepted = accepted.data_ptr()
    a.num_accepted = num_accepted.data_ptr()
    a.new_len = new_len.data_ptr() if new_len is not None else None
    a.status = status.data_ptr() if status is not None else None
    return a


def tree_kv_compact(k, v, prefix_len, max_prefix_len, parent, accepted, num_accepted, *,
                    page_table=None, page_size=0, new_len=None, status=None,
                    rope_theta=0.0, stream=None):
    """Move the accepted path's K/V rows to consecutive positions, in place (contiguous
    [B, S, Hkv, D] or paged pools with ``page_table``).  ``rope_theta`` > 0 also rotates
    every accepted key at its new position (the companion of the fused rotary embedding
    of ``tree_verify_attn``).  Returns ``(new_len, status)`` int32 [B] tensors (allocated
    when not given)."""
    torch = _torch()
    _require_cuda(k, v, prefix_len, parent, accepted, num_accepted, page_table, new_len, status)
    B = prefix_len.shape[0]
    dev = k.device
    with _on(stream):
        new_len = torch.empty(B, dtype=torch.int32, device=dev) if new_len is None else new_len
        status = torch.empty(B, dtype=torch.int32, device=dev) if status is None else status
    a = make_compact_args(k, v, prefix_len, max_prefix_len, parent, accepted, num_accepted,
                          page_table, page_size, new_len, status, rope_theta)
    _check(lib().tree_kv_compact(ctypes.byref(a), _stream(stream)))
    return new_len, status


class PreparedCall:
    """An after-pass entry point whose arguments are marshalled once: calling it only makes
    the C call (on the stream current at preparation, or the one given then) and returns
    ``result``, the output tensors.  It keeps every tensor it was made from alive; their
    contents may change between calls, their storage may not, and calls on one object
    share its outputs and workspace: the caller orders them."""

    def __init__(self, name, args, keep, stream, result):
        self._fn, self._a, self._keep, self._stream = getattr(lib(), name), args, keep, stream
        self._ref = ctypes.byref(args)
        self.result = result

    def __call__(self):
        _check(self._fn(self._ref, self._stream))
        return self.result


def _outputs(dev, stream, shapes, given):
    torch = _torch()
    with _on(stream):
        return tuple(torch.empty(sh, dtype=torch.int32, device=dev) if t is None else t
                     for sh, t in zip(shapes, given))


def prepare_tree_accept_greedy(logits, tokens, parent, target=None, accepted=None,
                               emitted=None, num_accepted=None, workspace=None, stream=None):
    """``tree_accept_greedy`` prepared once (same arguments); see :class:`PreparedCall`."""
    _require_cuda(logits, tokens, parent, target, accepted, emitted, num_accepted, workspace)
    B, N, _ = logits.shape
    outs = _outputs(logits.device, stream, ((B, N), (B, N), (B, N), (B,)),
                    (target, accepted, emitted, num_accepted))
    a = make_accept_args(logits, tokens, parent, *outs)
    need = int(lib().tree_accept_greedy_workspace_size(ctypes.byref(a)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        with _on(stream):
            workspace = _torch().empty(max(need, 16), dtype=_torch().uint8,
                                       device=logits.device)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    return PreparedCall("tree_accept_greedy", a, (logits, tokens, parent, workspace),
                        _stream(stream), outs)


def prepare_tree_accept_stochastic(p, q, tokens, parent, uniform, accepted=None,
                                   emitted=None, num_accepted=None, stream=None):
    """``tree_accept_stochastic`` prepared once (same arguments); see :class:`PreparedCall`."""
    _require_cuda(p, q, tokens, parent, uniform, accepted, emitted, num_accepted)
    B, N, _ = p.shape
    outs = _outputs(p.device, stream, ((B, N), (B, N), (B,)), (accepted, emitted, num_accepted))
    a = make_sample_args(p, q, tokens, parent, uniform, *outs)
    return PreparedCall("tree_accept_stochastic", a, (p, q, tokens, parent, uniform),
                        _stream(stream), outs)


def prepare_tree_kv_compact(k, v, prefix_len, max_prefix_len, parent, accepted, num_accepted,
                            *, page_table=None, page_size=0, new_len=None, status=None,
                            rope_theta=0.0, stream=None):
    """``tree_kv_compact`` prepared once (same arguments); see :class:`PreparedCall`.  Each
    call moves the rows the accepted lists name at that time, in place."""
    _require_cuda(k, v, prefix_len, parent, accepted, num_accepted, page_table, new_len, status)
    B = prefix_len.shape[0]
    outs = _outputs(k.device, stream, ((B,), (B,)), (new_len, status))
    a = make_compact_args(k, v, prefix_len, max_prefix_len, parent, accepted, num_accepted,
                          page_table, page_size, *outs, rope_theta)
    return PreparedCall("tree_kv_compact", a,
                        (k, v, prefix_len, parent, accepted, num_accepted, page_table),
                        _stream(stream), outs)


# ------------------------------------------------------------------ budget policy ----
def _probs(rank_prob):
    pr = np.ascontiguousarray(rank_prob, dtype=np.float64)
    if pr.ndim != 1:
        raise ValueError("rank_prob must be one-dimensional")
    return pr


def tree_expected_tokens(parent, rank, rank_prob):
    """Expected tokens per step of one tree under greedy verification.  Returns
    ``(expected, reach)`` with ``reach`` the per-node reach probabilities."""
    par = np.ascontiguousarray(parent, dtype=np.int32)
    rk = np.ascontiguousarray(rank, dtype=np.int32)
    if par.shape != rk.shape or par.ndim != 1:
        raise ValueError("parent and rank must be one-dimensional and of equal length")
    pr = _probs(rank_prob)
    reach = np.empty(max(par.size, 1), np.float64)
    out = ctypes.c_double(0.0)
    _check(lib().tree_expected_tokens(par.ctypes.data, rk.ctypes.data, par.size,
                                      pr.ctypes.data, pr.size, reach.ctypes.data,
                                      ctypes.byref(out)))
    return out.value, reach[:par.size].copy()


def tree_ridge_tokens(peak_flops, hbm_bytes_per_s, bytes_per_weight=2.0):
    """Tokens per step at which a decode step turns compute-bound."""
    out = ctypes.c_double(0.0)
    _check(lib().tree_ridge_tokens(float(peak_flops), float(hbm_bytes_per_s),
                                   float(bytes_per_weight), ctypes.byref(out)))
    return out.value


def tree_budget_nodes(batch, ridge_tokens, max_nodes=MAX_NODES):
    """Largest tree size N with batch * N <= ridge, within [1, max_nodes]."""
    out = ctypes.c_int32(0)
    _check(lib().tree_budget_nodes(int(batch), float(ridge_tokens), int(max_nodes),
                                   ctypes.byref(out)))
    return out.value


def _paths_from_csr(ranks, path_off, k):
    return [tuple(int(x) for x in ranks[path_off[i]:path_off[i + 1]]) for i in range(k)]


def tree_best_static(rank_prob, nodes, max_depth):
    """Best static tree of at most ``nodes`` nodes.  Returns ``(paths, expected)``, the
    rank paths in the builder's node order."""
    pr = _probs(rank_prob)
    cap = max(1, (int(nodes) - 1) * int(max_depth))
    ranks = np.empty(cap, np.int32)
    path_off = np.empty(max(1, int(nodes)), np.int64)
    k = ctypes.c_int32(0)
    e = ctypes.c_double(0.0)
    _check(lib().tree_best_static(pr.ctypes.data, pr.size, int(nodes), int(max_depth),
                                  ranks.ctypes.data, cap, path_off.ctypes.data,
                                  ctypes.byref(k), ctypes.byref(e)))
    return _paths_from_csr(ranks, path_off, k.value), e.value


def tree_budget_plan(batch, ridge_tokens, rank_prob, max_nodes=MAX_NODES, max_depth=8):
    """Tree size for the batch and the best static tree of that size.  Returns
    ``(nodes, paths, expected)``."""
    pr = _probs(rank_prob)
    n_cap = max(1, min(int(max_nodes), MAX_NODES))
    cap = max(1, (n_cap - 1) * int(max_depth))
    ranks = np.empty(cap, np.int32)
    path_off = np.empty(n_cap, np.int64)
    n = ctypes.c_int32(0)
    k = ctypes.c_int32(0)
    e = ctypes.c_double(0.0)
    _check(lib().tree_budget_plan(int(batch), float(ridge_tokens), int(max_nodes),
                                  pr.ctypes.data, pr.size, int(max_depth), ctypes.byref(n),
                                  ranks.ctypes.data, cap, path_off.ctypes.data,
                                  ctypes.byref(k), ctypes.byref(e)))
    return n.value, _paths_from_csr(ranks, path_off, k.value), e.value
