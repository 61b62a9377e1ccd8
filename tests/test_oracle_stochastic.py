"""Pins of the oracle's stochastic tree walk and inverse-CDF draw (CPU only).

Each pin comes from outside the oracle's own formulas: values printed on the pages (the
chain's expected tokens), a reduction to the already pinned greedy walk, special cases
whose outcome follows from the acceptance rule alone, and the property the rule exists
for -- the emitted tokens are distributed exactly as the target's own samples -- checked
end to end with a chi-square test that a planted mistake must fail.
"""
import json
import os

import numpy as np
import pytest

from oracle import accept as A
from oracle import meta as M
from tree_attention_draft_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "speculative_sampling_chain.json")

# upper 0.1% point of the chi-square distribution with 26 degrees of freedom
CHI2_26_999 = 54.05


# ---------------------------------------------------------------- inverse-CDF draw -----
@pytest.mark.parametrize("weights,u,want", [
    ([0.2, 0.3, 0.5], 0.0, 0),
    ([0.2, 0.3, 0.5], 0.19, 0),
    ([0.2, 0.3, 0.5], 0.21, 1),
    ([0.2, 0.3, 0.5], 0.49, 1),
    ([0.2, 0.3, 0.5], 0.51, 2),
    ([0.2, 0.3, 0.5], 0.999, 2),
    ([2.0, 3.0, 5.0], 0.51, 2),          # unnormalised weights
    ([0.0, 1.0, 0.0, 1.0], 0.0, 1),      # weight-zero entries are never drawn
    ([0.0, 1.0, 0.0, 1.0], 0.5, 3),
    ([1.0, 0.0, 0.0], 1.0 - 2.0 ** -53, 0),  # no running sum exceeds u * total
])
def test_inverse_cdf_hand_cases(weights, u, want):
    assert A.sample_inverse_cdf(weights, u) == want


def test_inverse_cdf_frequencies():
    w = np.array([0.1, 0.0, 0.45, 0.05, 0.4])
    rng = np.random.default_rng(5)
    n = 40000
    counts = np.bincount([A.sample_inverse_cdf(w, x) for x in rng.random(n)], minlength=5)
    assert counts[1] == 0
    keep = w > 0
    chi2 = (((counts - n * w) ** 2)[keep] / (n * w)[keep]).sum()
    assert chi2 < 18.47  # upper 0.1% point, 4 dof


@pytest.mark.parametrize("bad", [[], [0.0, 0.0], [0.5, -0.1], [np.nan, 1.0]])
def test_inverse_cdf_rejects_invalid_weights(bad):
    with pytest.raises(ValueError):
        A.sample_inverse_cdf(bad, 0.5)


# ------------------------------------------------------------------ helpers -----------
def tree_inputs(rng, parent, V, draw_from_q=True):
    """Random target and drafter rows for every node and children drawn from their
    parent's q (the setting the rule is exact for)."""
    N = len(parent)
    p = rng.random((N, V)) ** 3
    q = rng.random((N, V)) ** 3
    p /= p.sum(1, keepdims=True)
    q /= q.sum(1, keepdims=True)
    draft = np.zeros(N, np.int64)
    for c in range(1, N):
        draft[c] = rng.choice(V, p=q[parent[c]]) if draw_from_q else rng.integers(V)
    return p, q, draft


def random_parent(rng, N):
    return [-1] + [int(rng.integers(0, i)) for i in range(1, N)]


# ------------------------------------------------------------------ the walk ----------
def test_structure_of_every_walk():
    rng = np.random.default_rng(11)
    for trial in range(300):
        N = int(rng.integers(1, 20))
        parent = random_parent(rng, N)
        p, q, draft = tree_inputs(rng, parent, 6)
        acc, em = A.accept_stochastic(parent, draft, p, q, rng.random(N))
        assert A.is_root_path(parent, acc)
        assert len(em) == len(acc)
        assert em[:-1] == [int(draft[c]) for c in acc[1:]]
        depth = M.meta_from_parent(parent, 0)["depth"]
        assert len(acc) <= max(depth) + 1


def test_one_hot_targets_reduce_to_the_greedy_walk():
    # a one-hot target accepts exactly the first child carrying its token and never
    # anything else, and every residual stays on that token: the greedy walk on argmax p
    rng = np.random.default_rng(12)
    V = 5
    for trial in range(300):
        N = int(rng.integers(1, 24))
        parent = random_parent(rng, N)
        _, q, _ = tree_inputs(rng, parent, V)
        if trial % 3 == 0:
            q = np.eye(V)[rng.integers(V, size=N)]   # drafters that are sure of themselves
        y = rng.integers(V, size=N)
        p = np.eye(V)[y]
        draft = rng.integers(V, size=N)
        got = A.accept_stochastic(parent, draft, p, q, rng.random(N))
        want = A.accept_greedy(parent, draft, y)
        assert got == (want[0], [int(t) for t in want[1]])


def test_target_equal_to_drafter_accepts_every_first_child():
    rng = np.random.default_rng(13)
    for trial in range(200):
        N = int(rng.integers(2, 20))
        parent = random_parent(rng, N)
        p, _, draft = tree_inputs(rng, parent, 7)
        q = p.copy()
        for c in range(1, N):   # children drawn from q = p, so q(token) > 0
            draft[c] = rng.choice(7, p=q[parent[c]])
        acc, em = A.accept_stochastic(parent, draft, p, q, rng.random(N))
        table = A.child_table(parent)
        node, path = 0, [0]
        while table[node]:
            node = table[node][0]
            path.append(node)
        assert acc == path


def test_draft_token_the_drafter_gave_no_mass():
    parent = [-1, 0]
    q = np.array([[0.0, 1.0, 0.0], [1 / 3] * 3])
    draft = [0, 0]
    p_has = np.array([[0.2, 0.5, 0.3], [1 / 3] * 3])
    p_not = np.array([[0.0, 0.5, 0.5], [1 / 3] * 3])
    for u in (0.0, 0.5, 0.999):
        assert A.accept_stochastic(parent, draft, p_has, q, [0.3, u])[0] == [0, 1]
        assert A.accept_stochastic(parent, draft, p_not, q, [0.3, u])[0] == [0]


def test_chain_expected_tokens_as_printed():
    g = json.load(open(GOLDEN))
    p, q, K = np.array(g["p"]), np.array(g["q"]), g["drafts"]
    assert np.isclose(np.minimum(p, q).sum(), g["alpha"])
    parent = [-1] + list(range(K))
    rng = np.random.default_rng(14)
    n = 40000
    total = 0
    P, Q = np.tile(p, (K + 1, 1)), np.tile(q, (K + 1, 1))
    for _ in range(n):
        draft = np.concatenate([[0], rng.choice(4, size=K, p=q)])
        total += len(A.accept_stochastic(parent, draft, P, Q, rng.random(K + 1))[1])
    assert abs(total / n - g["expected_tokens"]) < 0.025


# ------------------------------------------------------------- losslessness -----------
SHAPE = [-1, 0, 0, 0, 1, 1, 2]   # three root candidates, two of them with children


def joint_of_three_tokens(rng, T, Qm, n):
    """Counts of the first three tokens emitted after token 0 by repeated draft-and-verify
    rounds: each round grows SHAPE from the last token (children drawn i.i.d. from the
    drafter's row of their parent's token), walks it, and continues from the last emitted
    token."""
    V = T.shape[0]
    counts = np.zeros((V, V, V))
    for _ in range(n):
        seq, last = [], 0
        while len(seq) < 3:
            tok = np.zeros(len(SHAPE), np.int64)
            tok[0] = last
            for c in range(1, len(SHAPE)):
                tok[c] = rng.choice(V, p=Qm[tok[SHAPE[c]]])
            _, em = A.accept_stochastic(SHAPE, tok, T[tok], Qm[tok], rng.random(len(SHAPE)))
            seq += em
            last = seq[-1]
        counts[seq[0], seq[1], seq[2]] += 1
    return counts


def chi2_against_target(counts, T):
    n = counts.sum()
    want = n * T[0][:, None, None] * T[:, :, None] * T[None, :, :]
    return (((counts - want) ** 2) / want).sum()


def markov_pair():
    T = np.array([[0.6, 0.3, 0.1], [0.2, 0.2, 0.6], [0.35, 0.45, 0.2]])
    Qm = np.array([[0.2, 0.5, 0.3], [0.5, 0.4, 0.1], [0.1, 0.3, 0.6]])
    return T, Qm


def test_emitted_tokens_follow_the_target_exactly():
    T, Qm = markov_pair()
    counts = joint_of_three_tokens(np.random.default_rng(15), T, Qm, 30000)
    assert chi2_against_target(counts, T) < CHI2_26_999


def test_negative_control_siblings_against_raw_target(monkeypatch):
    # the mistake the pages warn of: a rejected sibling's mass is not removed, so the
    # next sibling (and the correction) are judged against the raw target again
    monkeypatch.setattr(A, "_after_rejection", lambda r, z, qn: r)
    T, Qm = markov_pair()
    counts = joint_of_three_tokens(np.random.default_rng(15), T, Qm, 30000)
    assert chi2_against_target(counts, T) > 4 * CHI2_26_999


# ----------------------------------------------------- the residual in closed form -----
def closed_form_residuals(p, q, k):
    """max(p - S q, 0) after k rejections, S the sum of the earlier totals (unnormalised),
    a rejection whose residual has no mass leaving everything unchanged."""
    R, S = p.copy(), 0.0
    out = [R]
    for _ in range(k):
        Z = R.sum()
        nxt = np.maximum(p - (S + Z) * q, 0.0)
        if nxt.sum() > 0:
            S, R = S + Z, nxt
        out.append(R)
    return out


def iterated_residuals(p, q, k):
    r = p.copy()
    out = [r]
    for _ in range(k):
        r = A._after_rejection(r, r.sum(), q)
        out.append(r)
    return out


def residuals_agree(p, q, k):
    for a, b in zip(iterated_residuals(p, q, k), closed_form_residuals(p, q, k)):
        if not np.allclose(a / a.sum(), b / b.sum(), rtol=1e-12, atol=1e-15):
            return False
    return True


def test_iterated_residual_equals_the_closed_form_up_to_scale():
    # the normalised residual after k rejections is max(p - S_k q, 0) / its total, with S_k
    # the running sum of the unnormalised totals: an identity independent of the
    # oracle's iteration (the device walk evaluates this form)
    rng = np.random.default_rng(16)
    for trial in range(200):
        V = int(rng.integers(2, 40))
        p = rng.random(V) ** 3 * (0.5 + rng.random())   # unnormalised rows too
        q = rng.random(V) ** 3
        q /= q.sum()
        if trial % 10 == 0:
            # the no-mass corner a walk can reach: an unnormalised drafter row with excess
            # mass everywhere (q = r / z exactly is not one: its children are always accepted)
            q = 2.0 * p / p.sum()
        assert residuals_agree(p, q, int(rng.integers(1, 12)))


def test_negative_control_residual_without_normalising(monkeypatch):
    # a residual that subtracts q from the unnormalised r breaks the identity
    monkeypatch.setattr(A, "_after_rejection",
                        lambda r, z, qn: np.maximum(r - qn, 0.0)
                        if np.maximum(r - qn, 0.0).sum() > 0 else r)
    rng = np.random.default_rng(17)
    bad = 0
    for _ in range(50):
        V = int(rng.integers(4, 40))
        p = rng.random(V) ** 3 * 3.0
        q = rng.random(V) ** 3
        q /= q.sum()
        bad += not residuals_agree(p, q, 4)
    assert bad > 25
