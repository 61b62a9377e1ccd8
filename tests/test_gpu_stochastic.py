"""GPU parity of tree_accept_stochastic against the oracle's stochastic walk.

Both sides take every decision in float64 on the same float32 distributions and float64
uniforms; accepted nodes, emitted tokens and counts must agree exactly.  (Totals are
summed in different orders on the two sides, so a decision could in principle differ
when a uniform lands within rounding of its threshold: an event of probability ~1e-13
per decision, which no case here comes near.)
"""
import numpy as np
import pytest

import tree_attention_draft_amd as tv
from oracle import accept as oacc
from tree_attention_draft_amd import workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print("[stochastic]", *a, flush=True)


def make_inputs(seed, B, N, V, temperature=1.0, shared_tree=False, one_hot=False,
                p_equals_q=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    if shared_tree:
        parents = [workloads.random_parent(rng, N)] * B
    else:
        parents = [workloads.random_parent(rng, N) for _ in range(B)]
    p = workloads.random_distributions(rng, (B, N, V), temperature)
    q = p.copy() if p_equals_q else workloads.random_distributions(rng, (B, N, V), temperature)
    if one_hot:
        p = np.zeros_like(p)
        p[np.arange(B)[:, None], np.arange(N)[None], rng.integers(V, size=(B, N))] = 1.0
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        for c in range(1, N):
            # children drawn from their parent's drafter row (inverse CDF on a uniform)
            row = q[b, parents[b][c]].astype(np.float64)
            tokens[b, c] = min(int(np.searchsorted(np.cumsum(row), rng.random() * row.sum(),
                                                   side="right")), V - 1)
    if one_hot:  # make matches likely: half the children carry their parent's target token
        tgt = p.argmax(-1)
        for b in range(B):
            for c in range(1, N):
                if rng.random() < 0.5:
                    tokens[b, c] = tgt[b, parents[b][c]]
    u = rng.random((B, N))
    return parents, p, q, tokens, u


def run_gpu(parents, p, q, tokens, u, shared_tree=False):
    import torch
    dev = "cuda"
    par = torch.tensor(np.array(parents[:1] if shared_tree else parents, np.int32), device=dev)
    if shared_tree:
        par = par[0]
    acc, em, na = tv.tree_accept_stochastic(
        torch.from_numpy(p).to(dev), torch.from_numpy(q).to(dev),
        torch.from_numpy(tokens).to(dev), par, torch.from_numpy(u).to(dev))
    torch.cuda.synchronize()
    return acc.cpu().numpy(), em.cpu().numpy(), na.cpu().numpy()


def check(parents, p, q, tokens, u, acc, em, na):
    B, N, _ = p.shape
    lengths = []
    for b in range(B):
        want_acc, want_em = oacc.accept_stochastic(parents[b], tokens[b], p[b], q[b], u[b])
        A = len(want_acc)
        assert int(na[b]) == A, (b, int(na[b]), A)
        assert acc[b, :A].tolist() == want_acc, (b, acc[b, :A].tolist(), want_acc)
        assert em[b, :A].tolist() == want_em, (b, em[b, :A].tolist(), want_em)
        assert (acc[b, A:] == -1).all() and (em[b, A:] == -1).all()
        lengths.append(A)
    return lengths


@pytest.mark.parametrize("B,N,V,temp", [
    (16, 1, 50, 1.0),        # the root alone: one bonus draw
    (64, 10, 7, 1.0),        # a tiny vocabulary: many rejections per level
    (32, 33, 1000, 0.7),
    (16, 64, 3000, 1.5),     # the largest trees
    (4, 33, 128256, 1.0),    # a Llama-3-sized vocabulary
])
def test_random_trees_match_the_oracle(B, N, V, temp):
    say(f"B={B} N={N} V={V} T={temp}")
    parents, p, q, tokens, u = make_inputs(7000 + N + V, B, N, V, temp)
    lengths = check(parents, p, q, tokens, u, *run_gpu(parents, p, q, tokens, u))
    say("accepted lengths", lengths[:16])


def test_shared_tree_row():
    parents, p, q, tokens, u = make_inputs(7100, 12, 20, 500, shared_tree=True)
    check(parents, p, q, tokens, u, *run_gpu(parents, p, q, tokens, u, shared_tree=True))


def test_one_hot_targets_and_equal_distributions():
    parents, p, q, tokens, u = make_inputs(7200, 24, 17, 64, one_hot=True)
    check(parents, p, q, tokens, u, *run_gpu(parents, p, q, tokens, u))
    parents, p, q, tokens, u = make_inputs(7300, 24, 17, 64, p_equals_q=True)
    lengths = check(parents, p, q, tokens, u, *run_gpu(parents, p, q, tokens, u))
    assert max(lengths) > 2


def test_draft_tokens_the_drafter_gave_no_mass():
    parents, p, q, tokens, u = make_inputs(7400, 16, 12, 40)
    rng = np.random.default_rng(7400)
    for b in range(16):   # some children's tokens get zero drafter mass at their parent
        for c in range(1, 12):
            if rng.random() < 0.4:
                q[b, parents[b][c], tokens[b, c]] = 0.0
                if rng.random() < 0.5:
                    p[b, parents[b][c], tokens[b, c]] = 0.0
    check(parents, p, q, tokens, u, *run_gpu(parents, p, q, tokens, u))


def test_out_of_range_tokens_are_never_accepted():
    parents, p, q, tokens, u = make_inputs(7500, 8, 9, 30)
    tokens[:, 1::2] = 30 + np.arange(tokens[:, 1::2].shape[1])   # outside [0, V)
    acc, em, na = run_gpu(parents, p, q, tokens, u)
    for b in range(8):
        A = int(na[b])
        path = acc[b, :A].tolist()
        assert oacc.is_root_path(parents[b], path)
        assert all(n % 2 == 0 for n in path[1:])
        assert 0 <= em[b, A - 1] < 30


def test_empty_batch():
    import torch
    z = torch.zeros((0, 4, 10), dtype=torch.float32, device="cuda")
    acc, em, na = tv.tree_accept_stochastic(
        z, z, torch.zeros((0, 4), dtype=torch.int32, device="cuda"),
        torch.tensor([-1, 0, 0, 1], dtype=torch.int32, device="cuda"),
        torch.zeros((0, 4), dtype=torch.float64, device="cuda"))
    assert acc.shape == (0, 4) and na.shape == (0,)


def test_strided_rows_with_a_tail():
    # rows 16-byte aligned (stride 1004 entries) but V = 1001: the grouped loads take the
    # first 1000 entries of each row and the tail entry is read on its own
    import torch
    B, N, V, W = 6, 14, 1001, 1004
    parents, p, q, tokens, u = make_inputs(7600, B, N, V)
    wp = np.zeros((B, N, W), np.float32)
    wq = np.zeros((B, N, W), np.float32)
    wp[..., :V], wq[..., :V] = p, q
    dev = "cuda"
    tp = torch.from_numpy(wp).to(dev)[..., :V]
    tq = torch.from_numpy(wq).to(dev)[..., :V]
    assert tp.stride(1) == W
    acc, em, na = tv.tree_accept_stochastic(
        tp, tq, torch.from_numpy(tokens).to(dev),
        torch.tensor(np.array(parents, np.int32), device=dev), torch.from_numpy(u).to(dev))
    torch.cuda.synchronize()
    check(parents, p, q, tokens, u, acc.cpu().numpy(), em.cpu().numpy(), na.cpu().numpy())
