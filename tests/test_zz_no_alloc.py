"""tree_verify_attn_static (the entry point that allocates nothing) against
tree_verify_attn, through the C ABI, on two calls in a row -- the second with a smaller
input -- each also checked against the fp64 oracle.  Both calls split the keys, so the
static device array carries the partials; the second call must not see anything the
first one left in it."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import tree_attention_draft_amd as tv  # noqa: E402
from tree_attention_draft_amd import workloads  # noqa: E402

from gpu_cases import Case, say  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def trees(seed, B, n, cap):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [workloads.random_tree(rng, n, cap)[0] for _ in range(B)]


def static_call(c, out, lse, **kw):
    """Both entry points through ctypes with the same argument struct."""
    d = c.device()
    a = tv.make_args(d["q"], d["k"], d["v"], d["parent"], d["prefix_len"], int(c.L.max()),
                     out=out, lse=lse, **kw)
    need = tv.lib().tree_verify_attn_workspace_size(ctypes.byref(a))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = tv.lib().tree_verify_attn_static(ctypes.byref(a), stream)
    assert st == 0, tv.lib().tv_last_error().decode()
    torch.cuda.synchronize()
    return need


def reference_call(c, **kw):
    d = c.device()
    out, lse = tv.tree_verify_attn(d["q"], d["k"], d["v"], d["parent"], d["prefix_len"],
                                   int(c.L.max()), **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("kind", ["mfma", "mfma_many_splits", "mfma_paged", "valu_f32"])
def test_static_entry_point_two_calls(kind):
    if kind == "mfma":
        big = Case("static_big", [3000, 1500, 64, 2500, 777], trees=trees(7701, 5, 33, 8),
                   seed=7702)
        small = Case("static_small", [900, 40], trees=trees(7703, 2, 17, 6), seed=7704)
        kw_big, kw_small = dict(num_splits=6), dict(num_splits=3)
    elif kind == "mfma_many_splits":
        # 40 and 12 splits: the merge spreads each output over 8, then 2, thread groups
        big = Case("static_many", [3000, 2500], trees=trees(7711, 2, 33, 8), seed=7712)
        small = Case("static_many_small", [900, 40], trees=trees(7713, 2, 17, 6), seed=7714)
        kw_big, kw_small = dict(num_splits=40), dict(num_splits=12)
    elif kind == "mfma_paged":
        # paged KV (pages of 16): eight splits of five requests run one team per workgroup
        # and the vector page addresses, three splits of two requests two teams and the
        # scalar ones
        big = Case("static_paged", [3000, 1500, 64, 2500, 777], trees=trees(7715, 5, 33, 8),
                   seed=7716, page_size=16, page_seed=7717)
        small = Case("static_paged_small", [900, 40], trees=trees(7718, 2, 33, 8), seed=7719,
                     page_size=16, page_seed=7720)
        kw_big = dict(num_splits=8, page_table=big.device()["page_table"], page_size=16)
        kw_small = dict(num_splits=3, page_table=small.device()["page_table"], page_size=16)
    else:
        big = Case("static_big_f32", [700, 333, 1200], trees=trees(7705, 3, 20, 6), Hq=8,
                   Hkv=2, dtype="f32", seed=7706)
        small = Case("static_small_f32", [90], trees=trees(7707, 1, 10, 4), Hq=4, Hkv=2,
                     D=64, dtype="f32", seed=7708)
        kw_big, kw_small = dict(num_splits=5), dict(num_splits=2)
    for c, kw in ((big, kw_big), (small, kw_small)):
        d = c.device()
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full((c.B, c.N, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
        need = static_call(c, out, lse, **kw)
        assert 0 < need <= tv.STATIC_SCRATCH_BYTES
        say(c.name, f"static call used {need} bytes of the static array")
        ref_out, ref_lse = reference_call(c, **kw)
        # the same kernels and plan: bit-identical to the allocating entry point
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        c.check(out.float().cpu().numpy().astype(np.float64),
                lse.cpu().numpy().astype(np.float64))


def test_static_entry_point_rejects_oversized_plans_before_enqueueing():
    c = Case("static_reject", [4000] * 4, trees=trees(7709, 4, 33, 8), seed=7710)
    d = c.device()
    out = torch.full_like(d["q"], 3.0)
    a = tv.make_args(d["q"], d["k"], d["v"], d["parent"], d["prefix_len"], 4000, out=out,
                     num_splits=63)
    need = tv.lib().tree_verify_attn_workspace_size(ctypes.byref(a))
    assert need > tv.STATIC_SCRATCH_BYTES
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert tv.lib().tree_verify_attn_static(ctypes.byref(a), stream) == 6  # TV_ERR_WORKSPACE
    assert "static scratch" in tv.lib().tv_last_error().decode()
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())       # nothing was enqueued


def test_static_entry_point_replays_in_a_captured_graph():
    # the callers this entry point is for: code under graph capture.  A split plan (so the
    # static array and the merge kernel are inside the graph) is captured once and replayed
    # three times, with new queries written eagerly between replays; every replay must
    # equal an eager tree_verify_attn call on the same inputs bit for bit.
    c = Case("graph", [600, 333, 97], trees=trees(9200, 3, 33, 8), seed=9200)
    d = c.device()
    q, maxl = d["q"], int(c.L.max())
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    kw = dict(out=out, lse=lse, num_splits=3)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first call outside capture: module load, array address
        tv.tree_verify_attn_static(q, d["k"], d["v"], d["parent"], d["prefix_len"], maxl, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tv.tree_verify_attn_static(q, d["k"], d["v"], d["parent"], d["prefix_len"], maxl, **kw)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9201)
    for rep in range(3):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = tv.tree_verify_attn(q, d["k"], d["v"], d["parent"], d["prefix_len"],
                                           maxl, num_splits=3)
        torch.cuda.synchronize()
        say("graph replay", rep, "max |diff|", float((got_o.float() - ref_o.float()).abs().max()))
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), rep
