"""Pins for the oracle's acceptance walks and its Philox (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import accept, marginal, philox

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    kat = json.load(open(os.path.join(GOLD, "philox_kat.json")))
    for case in kat["cases"]:
        ctr = [int(x, 16) for x in case["ctr"]]
        key = [int(x, 16) for x in case["key"]]
        out = [int(x, 16) for x in case["out"]]
        assert list(philox.philox4x32_10(ctr, key)) == out
        vb = philox.philox_batch([ctr[0]], [ctr[1]], [ctr[2]], [ctr[3]], key[0], key[1])
        assert [int(v[0]) for v in vb] == out


def one_child_tree(tok):
    return [-1, 0], [-1, tok], [0, 1]


def test_worked_example_closed_form():
    """Course notes, three-token example: q = (.1, .1, .8), p = (.2, .4, .4)."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    q, p = np.array(g["q"]), np.array(g["p"])
    target = np.log(np.stack([p, p]))      # rows for the root and the child
    draft = np.log(q)[None, :]
    mix = np.zeros(3)
    for x in range(3):
        par, tok, dep = one_child_tree(x)
        tab = accept.ResidualTables(par, tok, dep, target, draft, 1.0)
        a = min(1.0, tab.pc[0][0] / tab.qc[0][0])
        assert abs(a - g["accept_prob"][x]) < 1e-12
        stop, reach = accept.exact_outcomes(tab)
        assert abs(reach[1] - a) < 1e-12 and abs(stop[0] - (1 - a)) < 1e-12
        if x == 2:
            np.testing.assert_allclose(tab.final[0], g["residual"], atol=1e-12)
        # output law when x was proposed: accept -> x, reject -> residual
        mix += q[x] * (a * np.eye(3)[x] + (1 - a) * tab.final[0])
    np.testing.assert_allclose(mix, g["output"], atol=1e-12)
    assert abs(np.sum(np.maximum(p - q, 0)) - g["deficit_total"]) < 1e-12
    assert abs(q[2] * (1 - g["accept_prob"][2]) - g["rejected_mass"]) < 1e-12


def test_worked_example_sampled_frequencies():
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    q, p = np.array(g["q"]), np.array(g["p"])
    par, tok, dep = one_child_tree(2)
    tab = accept.ResidualTables(par, tok, dep, np.log(np.stack([p, p])), np.log(q)[None, :], 1.0)
    n = 20000
    res = [accept.walk_sampled(tab, dep, 0x5EED5EED, t, 0) for t in range(n)]
    acc = np.mean([r[0] == 1 for r in res])
    assert abs(acc - 0.5) < 3.5 * math.sqrt(0.25 / n)
    rej = [r[2] for r in res if r[0] == 0]
    fa = np.mean([x == 0 for x in rej])
    assert abs(fa - 0.25) < 3.5 * math.sqrt(0.25 * 0.75 / len(rej))
    assert all(x != 2 for x in rej)


def test_degenerate_cases():
    rng = np.random.default_rng(1)
    z = rng.standard_normal(20)
    par, tok, dep = [-1, 0, 0], [-1, 3, 7], [0, 1, 1]
    # p = q: never reject, and no NaN from an empty residual
    tab = accept.ResidualTables(par, tok, dep, np.stack([z, z, z]), z[None, :], 1.0)
    stop, reach = accept.exact_outcomes(tab)
    assert reach[1] == pytest.approx(1.0) and stop[0] == 0.0
    assert np.all(np.isfinite(tab.final[0]))
    # p(x) = 0 < q(x): always reject token 3 (target logit far below the rest)
    zt = z.copy()
    zt[3] = -1e4
    tab = accept.ResidualTables(par, tok, dep, np.stack([zt, zt, zt]), z[None, :], 1.0)
    stop, reach = accept.exact_outcomes(tab)
    assert reach[1] == 0.0
    for t in range(200):
        assert accept.walk_sampled(tab, dep, 1, t, 0)[1] != 1


def test_greedy_walk_follows_argmax_chain_and_ties():
    rng = np.random.default_rng(2)
    L, V = 6, 40
    z = rng.standard_normal((L, V)) * 2
    t = marginal.build_marginal(z, 0, 25, 0.0)
    target = np.stack([z[min(t.depth[j], L - 1)] for j in range(t.n + 1)])
    alen, node, nxt = accept.walk_greedy(t.parent, t.token, t.depth, target)
    chain = [int(np.argmax(z[d])) for d in range(L)]
    # the accepted path is the longest prefix of the argmax chain present in the tree
    paths = set(t.paths())
    k = 0
    while k < L and tuple(chain[:k + 1]) in paths:
        k += 1
    assert alen == k and nxt == chain[min(k, L - 1)]
    # equal maxima: the smaller id wins
    row = np.zeros((1, 10))
    row[0, [4, 2, 8]] = 5.0
    assert accept.walk_greedy([-1], [-1], [0], row)[2] == 2


def test_yield_bounds_and_total_probability():
    rng = np.random.default_rng(3)
    L, V = 5, 30
    z = rng.standard_normal((L, V)) * 2
    t = marginal.build_marginal(z, 0, 18, 0.0)
    target = np.stack([z[min(t.depth[j], L - 1)] + rng.standard_normal(V) for j in range(t.n + 1)])
    tab = accept.ResidualTables(t.parent, t.token, t.depth, target, z, 1.0)
    stop, _ = accept.exact_outcomes(tab)
    assert abs(stop.sum() - 1.0) < 1e-12
    for tr in range(300):
        alen, node, nxt = accept.walk_sampled(tab, t.depth, 7, tr, 0)
        assert 0 <= alen <= max(t.depth) and t.depth[node] == alen
        assert 0 <= nxt < V
        # committed tokens per round: accepted drafts plus one extra token
        assert 1 <= alen + 1 <= L + 1


def match_case(seed=21, L=4, V=12, B=14):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((L, V)) * 1.5
    t = marginal.build_marginal(z, 0, B, 0.0)
    target = np.stack([z[min(t.depth[j], L - 1)] + rng.standard_normal(V) for j in range(t.n + 1)])
    return t, target


def test_match_law_is_lossless():
    """Target-sample matching commits exact target samples: whatever the tree, the first
    committed token (a depth-1 child's token, or the token emitted at the root) has the law
    p_root, and after a child c it continues with p_c, which is what the law's reach/stop
    split must reproduce token by token."""
    t, target = match_case()
    for T in (1.0, 0.7):
        stop, reach, emit = accept.match_outcomes(t.parent, t.token, target, T)
        assert abs(stop.sum() - 1.0) < 1e-12
        kids = accept.children_lists(t.parent)
        for j in range(t.n + 1):
            if reach[j] == 0.0:
                continue
            p = accept.softmax_row(target[j], T)
            law = np.zeros_like(p)       # next committed token, given the walk reached j
            if emit[j] is not None:
                law += stop[j] / reach[j] * emit[j]
            for c in kids[j]:
                law[t.token[c]] += reach[c] / reach[j]
            np.testing.assert_allclose(law, p, atol=1e-12)


def test_match_walk_frequencies():
    t, target = match_case(seed=22)
    stop, _, emit = accept.match_outcomes(t.parent, t.token, target, 1.0)
    n = 20000
    res = [accept.walk_match(t.parent, t.token, t.depth, target, 1.0, 0x5EED5EED, tr, 3) for tr in range(n)]
    nodes = np.bincount([r[1] for r in res], minlength=t.n + 1)
    for j in range(t.n + 1):
        assert abs(nodes[j] - n * stop[j]) <= 3.5 * math.sqrt(n * stop[j] * (1 - stop[j])) + 1
    j = int(np.argmax(stop))
    toks = np.array([r[2] for r in res if r[1] == j])
    m = toks.shape[0]
    for v in range(target.shape[1]):
        f = emit[j][v]
        assert abs(np.sum(toks == v) - m * f) <= 3.5 * math.sqrt(m * f * (1 - f)) + 1
    for alen, node, nxt in res[:200]:
        assert t.depth[node] == alen and nxt not in [t.token[c] for c in accept.children_lists(t.parent)[node]]


def test_match_walk_sharp_target_is_greedy():
    """A target row with one dominant logit draws that token with probability ~1: the walk
    then follows the greedy walk exactly."""
    t, target = match_case(seed=23)
    sharp = target.copy()
    for j in range(sharp.shape[0]):
        sharp[j, int(np.argmax(sharp[j]))] += 80.0
    g = accept.walk_greedy(t.parent, t.token, t.depth, sharp)
    for tr in range(50):
        assert accept.walk_match(t.parent, t.token, t.depth, sharp, 1.0, 9, tr, 0) == g


def _multichild():
    g = json.load(open(os.path.join(GOLD, "multichild_example.json")))
    tr = g["tree"]
    target = np.log(np.array(g["target_rows"]))
    draft = np.log(np.array(g["draft_rows"]))
    return g, tr["parent"], tr["token"], tr["depth"], target, draft


def _frac(x):
    return x[0] / x[1]


def test_multichild_closed_form():
    """A node with three children and one with two, on two depths with different draft rows:
    the sibling-by-sibling residual (q fixed per node, renormalised after every rejection)
    against fractions worked by hand. Updating p' with the other depth's draft row, skipping
    a renormalisation or keeping p instead of the residual each changes an acceptance
    probability below."""
    g, par, tok, dep, target, draft = _multichild()
    tab = accept.ResidualTables(par, tok, dep, target, draft, 1.0)
    for c, want in g["accept_prob"].items():
        c = int(c)
        j = par[c]
        i = tab.kids[j].index(c)
        a = min(1.0, tab.pc[j][i] / tab.qc[j][i])
        assert abs(a - _frac(want)) < 1e-12, (c, a)
    stop, reach = accept.exact_outcomes(tab)
    np.testing.assert_allclose(reach, [_frac(x) for x in g["reach"]], atol=1e-12)
    np.testing.assert_allclose(stop, [_frac(x) for x in g["stop"]], atol=1e-12)
    assert abs(np.sum(stop) - 1.0) < 1e-12
    for j, want in g["final_residual"].items():
        np.testing.assert_allclose(tab.final[int(j)], [_frac(x) for x in want], atol=1e-12)
    # leaves draw from their own target distribution
    for j in (2, 3, 4, 5):
        np.testing.assert_allclose(tab.final[j], np.array(g["target_rows"][j]), atol=1e-12)


def test_multichild_sampled_against_hand_law():
    """The sampled walk's stop frequencies over 20,000 Philox trials against the hand law."""
    g, par, tok, dep, target, draft = _multichild()
    tab = accept.ResidualTables(par, tok, dep, target, draft, 1.0)
    n = 20000
    nodes = np.array([accept.walk_sampled(tab, dep, 0x5EED5EED, t, 3)[1] for t in range(n)])
    for j, want in enumerate(g["stop"]):
        p = _frac(want)
        f = np.mean(nodes == j)
        assert abs(f - p) <= 4 * math.sqrt(max(p * (1 - p), 1e-12) / n) + 1e-12, (j, f, p)


def test_walk_margin_is_distance_to_the_decision():
    """The margin the oracle reports for a walk is the smallest |u q - p'| over its tests and
    the draw's distance to its CDF boundaries: recomputed from the same uniforms."""
    g, par, tok, dep, target, draft = _multichild()
    tab = accept.ResidualTables(par, tok, dep, target, draft, 1.0)
    for t in range(50):
        res, m = accept.walk_sampled_margin(tab, dep, 0x5EED5EED, t, 0)
        assert res == accept.walk_sampled(tab, dep, 0x5EED5EED, t, 0)
        assert 0.0 <= m <= 1.0
    # a draw exactly on a boundary has margin 0; one in the middle of a token has margin > 0
    p = np.array([0.25, 0.25, 0.5])
    assert accept.inverse_cdf_margin(p, 0.5, 2) == 0.0
    assert abs(accept.inverse_cdf_margin(p, 0.75, 2) - 0.25) < 1e-15


def test_match_walk_margin_agrees_with_walk():
    g, par, tok, dep, target, draft = _multichild()
    for t in range(30):
        res, m = accept.walk_match_margin(par, tok, dep, target, 1.0, 0x5EED5EED, t, 1)
        assert res == accept.walk_match(par, tok, dep, target, 1.0, 0x5EED5EED, t, 1)
        assert 0.0 <= m <= 0.5
