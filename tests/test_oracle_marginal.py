"""Pins for the oracle's marginal Top-B tree (CPU only).

Brute force over the whole vocabulary, the S_K restriction, Lemma 1 (heap ==
sort), special cases that reduce to a plain argmax / top-B, prefix closure,
and Proposition 1 of DDTree by Monte Carlo.
"""
import math

import numpy as np
import pytest

import synth
from oracle import accept, marginal, rowsweep, treeout


def tree_key(t):
    return [(p, s) for p, s in zip(t.paths()[1:], t.score[1:])]


def same_tree(a, b, atol=0.0):
    pa, pb = a.paths(), b.paths()
    assert pa == pb
    assert a.parent == b.parent and a.depth == b.depth
    np.testing.assert_allclose(a.score, b.score, rtol=0, atol=atol)


@pytest.mark.parametrize("r", range(4))
def test_tiny_config_heap_equals_full_vocab_brute_force(r):
    """Tiny marginal config (R=4, L=4, V=32, K=B=8, beta=0): every <=4-token prefix over the
    whole vocabulary (1,082,400 per round) is scored and sorted; the top 8 must be exactly the
    DDTree heap's output over S_K with K = min(B, V) = 8."""
    z = rowsweep.as_f64(synth.tiny_marginal(), "f32")[r]
    heap_t = marginal.build_marginal(z, 8, 8, 0.0)
    brute_t = marginal.brute_force(z, 8, 0.0)
    same_tree(heap_t, brute_t)
    treeout.check_invariants(heap_t, 8, 4)
    assert heap_t.n == 8


@pytest.mark.parametrize("B", range(1, 15))
def test_two_token_vocab_depth_three(B):
    """DDTree blog checklist: brute-force a tiny case (2-token vocabulary, depth 3)."""
    rng = np.random.default_rng(100 + B)
    z = rng.standard_normal((3, 2))
    same_tree(marginal.build_marginal(z, 2, B, 0.0), marginal.brute_force(z, B, 0.0))


@pytest.mark.parametrize("beta", [0.0, -0.3, -2.0])
def test_heap_equals_brute_force_with_depth_bonus(beta):
    rng = np.random.default_rng(7)
    z = rng.standard_normal((3, 9)) * 2.0
    for B in (1, 5, 20, 60):
        same_tree(marginal.build_marginal(z, 9, B, beta), marginal.brute_force(z, B, beta))


def test_bf16_exact_ties_brute_force():
    """Heavily tied bf16 rows: the explicit tie-break must pick the same tree both ways."""
    b = synth.tie_rows(6, 3, seed=5)
    z = rowsweep.as_f64(b, "bf16")
    for B in (3, 10, 40, 100):
        same_tree(marginal.build_marginal(z, 6, B, 0.0), marginal.brute_force(z, B, 0.0))


def test_special_cases():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((5, 50)) * 3.0
    # B = 1: the argmax of the first position
    t = marginal.build_marginal(z, 0, 1, 0.0)
    assert t.n == 1 and t.token[1] == int(np.argmax(z[0]))
    # K = 1, B <= L: the argmax chain
    t = marginal.build_marginal(z, 1, 4, 0.0)
    assert t.token[1:] == [int(np.argmax(z[d])) for d in range(4)]
    assert t.parent[1:] == [0, 1, 2, 3]
    # L = 1: the top-B of one log-softmax row
    t = marginal.build_marginal(z[:1], 0, 7, 0.0)
    order = np.argsort(-z[0], kind="stable")[:7]
    assert t.token[1:] == list(order)
    ref_lp = z[0] - (np.max(z[0]) + np.log(np.sum(np.exp(z[0] - np.max(z[0])))))
    np.testing.assert_allclose(t.score[1:], ref_lp[order], atol=1e-12)
    # a huge depth penalty with B <= K keeps only depth-1 nodes
    t = marginal.build_marginal(z, 10, 6, -1e6)
    assert all(d == 1 for d in t.depth[1:]) and t.token[1:] == list(np.argsort(-z[0], kind="stable")[:6])


def test_positive_beta_rejected():
    with pytest.raises(ValueError):
        marginal.build_marginal(np.zeros((2, 4)), 2, 2, 0.5)


def test_invariants_ddtree_shape_small():
    b = synth.ddtree_logits(seed=2, R=2, L=16, V=3000)
    z = rowsweep.as_f64(b, "bf16")
    for r in range(2):
        t = marginal.build_marginal(z[r], 64, 64, 0.0)
        treeout.check_invariants(t, 64, 16)
        assert t.n == 64
        # mask rows: popcount = depth + 1, and each row contains its parent's row
        m = treeout.ancestor_mask(t.parent, 64)
        for i in range(1, t.n + 1):
            bits = sum(bin(int(w)).count("1") for w in m[i])
            assert bits == t.depth[i] + 1
            assert np.all((m[i] & m[t.parent[i]]) == m[t.parent[i]])


def test_literal_successor_rule_misses_prefixes():
    """Planted mistake in the oracle: the blog's literal rule (first child only when the
    last rank is the top one) loses prefixes that brute force finds."""
    rng = np.random.default_rng(11)
    z = rng.standard_normal((3, 6)) * 0.3   # flat rows: deep low-rank prefixes matter
    B = 30
    ref = marginal.brute_force(z, B, 0.0)
    lse = np.array([rowsweep.logsumexp_row(z[d]) for d in range(3)])
    ranks = np.stack([rowsweep.rank_order(z[d]) for d in range(3)])
    zk = np.take_along_axis(z, ranks, axis=1)
    import heapq
    Lsum = marginal.lse_prefix_sums(lse)
    heap = [(-(zk[0, 0] - Lsum[1]), (0,))]
    got = []
    while heap and len(got) < B:
        _, desc = heapq.heappop(heap)
        got.append(desc)
        d = len(desc)
        Z = sum(zk[i, desc[i]] for i in range(d))
        if d < 3 and desc[-1] == 0:
            heapq.heappush(heap, (-(Z + zk[d, 0] - Lsum[d + 1]), desc + (0,)))
        if desc[-1] + 1 < 6:
            sib = desc[:-1] + (desc[-1] + 1,)
            Zs = sum(zk[i, sib[i]] for i in range(d))
            heapq.heappush(heap, (-(Zs - Lsum[d]), sib))
    got_paths = {tuple(int(ranks[i, r]) for i, r in enumerate(desc)) for desc in got}
    assert got_paths != set(ref.paths()[1:])


def test_ancestor_mask_matches_hand_drawn_depth3():
    rows = []
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "mask_depth3.txt")
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([int(c) for c in line])
    parent = [-1, 0, 0, 1, 1, 2, 3]
    m = treeout.ancestor_mask(parent, 6)
    for i, row in enumerate(rows):
        bits = [(int(m[i, j >> 5]) >> (j & 31)) & 1 for j in range(7)]
        assert bits == row


def test_proposition1_expected_acceptance():
    """DDTree Proposition 1 (DARTree background; DDTree blog 2.1): if the target's greedy
    continuation Y is drawn from the factorised draft q_par, the mean accepted length of
    the greedy walk equals sum over tree nodes of q(u) = exp(s_0(u))."""
    rng = np.random.default_rng(21)
    L, V, B = 5, 12, 20
    z = rng.standard_normal((L, V)) * 1.5
    t = marginal.build_marginal(z, 0, B, 0.0)
    expect = sum(math.exp(s) for s in t.score[1:])
    probs = np.stack([np.exp(z[d] - rowsweep.logsumexp_row(z[d])) for d in range(L)])
    n = 20000
    acc = np.empty(n)
    onehot = np.full((t.n + 1, V), -10.0)
    for k in range(n):
        Y = [rng.choice(V, p=probs[d]) for d in range(L)]
        for j in range(t.n + 1):
            onehot[j].fill(-10.0)
            onehot[j, Y[min(t.depth[j], L - 1)]] = 0.0
        acc[k] = accept.walk_greedy(t.parent, t.token, t.depth, onehot)[0]
    se = acc.std() / math.sqrt(n)
    assert abs(acc.mean() - expect) < 3.5 * se + 1e-9, (acc.mean(), expect, se)
