"""GPU parity: tree verification walks (a7) against the oracle, on oracle-built trees."""
import json
import math
import os

import numpy as np
import pytest
import torch

import draft_tree_construction_amd as dt
import synth
from oracle import accept, marginal, rowsweep
from parity_util import dev_bf16, dev_f32, oracle_to_device

pytestmark = pytest.mark.gpu
SEED = synth.PHILOX_SEED
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def verification_case(R, L, V, B, seed=2):
    draft = synth.ddtree_logits(seed=seed, R=R, L=L, V=V)
    trees = [marginal.build_marginal(rowsweep.as_f64(draft[r], "bf16"), 0 if B <= 64 else 64, B, 0.0)
             for r in range(R)]
    depth = np.stack([t.arrays(B)[2] for t in trees])
    target = synth.verification_target(draft, depth, seed=5)
    return draft, trees, target


def host_outs(outs):
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


@pytest.mark.parametrize("R,L,V,B", [(8, 16, 5000, 64), (4, 5, 300, 20), (3, 16, 151936, 64)])
def test_greedy_walk_matches_oracle(R, L, V, B):
    draft, trees, target = verification_case(R, L, V, B)
    dtree = oracle_to_device(trees, B)
    alen, anode, nxt = host_outs(dt.accept_tree(dtree, dev_bf16(target), None, 0.0, SEED, 0, 3))
    for r in range(R):
        ref = accept.walk_greedy(trees[r].parent, trees[r].token, trees[r].depth,
                                 rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16"))
        for t in range(3):
            assert (alen[t, r], anode[t, r], nxt[t, r]) == ref


def test_greedy_walk_noise_free_target_follows_argmax_chain():
    R, L, V, B = 4, 16, 3000, 64
    draft = synth.ddtree_logits(seed=9, R=R, L=L, V=V)
    trees = [marginal.build_marginal(rowsweep.as_f64(draft[r], "bf16"), 0, B, 0.0) for r in range(R)]
    target = np.stack([draft[r, np.minimum(t.arrays(B)[2].clip(0), L - 1)] for r, t in enumerate(trees)])
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, B), dev_bf16(target), None, 0.0, SEED))
    for r in range(R):
        z = rowsweep.as_f64(draft[r], "bf16")
        chain = [int(np.argmax(z[d])) for d in range(L)]
        paths = set(trees[r].paths())
        k = 0
        while k < L and tuple(chain[:k + 1]) in paths:
            k += 1
        assert alen[0, r] == k and nxt[0, r] == chain[min(k, L - 1)]


def test_sampled_walk_lazy_equals_tables():
    """One trial per call (the cooperative walk, four workgroups per round) and many trials
    per call (the table walk) agree for the same trial index: the exact C values are equal,
    and the LSE and draw prefix, summed in another order, can only move a decision that sits
    within float rounding of its threshold."""
    R, L, V, B = 6, 16, 4000, 64
    draft, trees, target = verification_case(R, L, V, B)
    dtree = oracle_to_device(trees, B)
    tg, dr = dev_bf16(target), dev_bf16(draft)
    many = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, 0, 64))
    bad = 0
    for t in range(0, 64, 3):
        one = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, t, 1))
        bad += int(np.sum(np.any(np.stack([one[k][0] != many[k][t] for k in range(3)]), axis=0)))
    assert bad <= 1, bad


def test_sampled_walk_trial_by_trial_against_oracle():
    R, L, V, B = 4, 16, 2000, 64
    draft, trees, target = verification_case(R, L, V, B)
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, B), dev_bf16(target), dev_bf16(draft),
                                                1.0, SEED, 0, 300))
    bad = 0
    for r in range(R):
        tab = accept.ResidualTables(trees[r].parent, trees[r].token, trees[r].depth,
                                    rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16"),
                                    rowsweep.as_f64(draft[r], "bf16"), 1.0)
        for t in range(300):
            ref = accept.walk_sampled(tab, trees[r].depth, SEED, t, r)
            bad += ref != (alen[t, r], anode[t, r], nxt[t, r])
    assert bad <= 2, bad   # decisions within float rounding of a threshold may differ


def test_sampled_walk_frequencies_within_3_sigma():
    """Accept-node frequencies over 10^6 seeded trials per round against the oracle's exact law."""
    R, L, V, B = 4, 16, 3000, 64
    n = 1_000_000
    draft, trees, target = verification_case(R, L, V, B, seed=12)
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, B), dev_bf16(target), dev_bf16(draft),
                                                1.0, SEED, 0, n))
    bins = beyond = 0
    for r in range(R):
        tab = accept.ResidualTables(trees[r].parent, trees[r].token, trees[r].depth,
                                    rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16"),
                                    rowsweep.as_f64(draft[r], "bf16"), 1.0)
        stop, _ = accept.exact_outcomes(tab)
        counts = np.bincount(anode[:, r], minlength=len(stop))
        for j, p in enumerate(stop):
            if p * n < 5:
                assert counts[j] <= max(10, 10 * p * n)
                continue
            bins += 1
            sig = math.sqrt(n * p * (1 - p))
            beyond += abs(counts[j] - n * p) > 3 * sig
        # extra-token law at the most frequent stopping node
        j = int(np.argmax(stop))
        sel = nxt[anode[:, r] == j, r]
        m = sel.shape[0]
        f = tab.final[j]
        for v in np.argsort(-f)[:5]:
            if f[v] * m < 5:
                continue
            bins += 1
            beyond += abs(np.sum(sel == v) - m * f[v]) > 3 * math.sqrt(m * f[v] * (1 - f[v]))
        assert np.all((alen[:, r] >= 0) & (alen[:, r] <= L))
    assert beyond <= 0.01 * bins + 2, (beyond, bins)


def test_worked_example_on_gpu():
    """Course notes' three-token example: q = (.1, .1, .8), p = (.2, .4, .4); one-child trees
    with child A, B, C; 10^6 trials each."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    q, p = np.array(g["q"]), np.array(g["p"])
    trees = []
    from oracle.treeout import Tree
    for x in range(3):
        t = Tree()
        t.add(0, x, 1, float(np.log(q[x])))
        trees.append(t)
    target = np.log(np.stack([[p, p]] * 3)).astype(np.float32)          # [3, 2, 3]
    draft = np.log(np.stack([[q]] * 3)).astype(np.float32)              # [3, 1, 3]
    n = 1_000_000
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, 1), dev_f32(target), dev_f32(draft), 1.0,
                                                SEED, 0, n))
    acc = alen.mean(axis=0)
    for x in range(3):
        a = g["accept_prob"][x]
        assert abs(acc[x] - a) <= 3 * math.sqrt(a * (1 - a) / n) + 1e-12
    rej = nxt[alen[:, 2] == 0, 2]
    for v, want in enumerate(g["residual"]):
        m = rej.shape[0]
        assert abs(np.mean(rej == v) - want) <= 3 * math.sqrt(want * (1 - want) / m) + 1e-12
    # the mixture over proposals x ~ q reproduces p
    out = np.zeros(3)
    for x in range(3):
        toks = np.where(alen[:, x] == 1, x, nxt[:, x])
        out += q[x] * np.bincount(toks, minlength=3) / n
    assert np.all(np.abs(out - p) <= 3 * np.sqrt(p * (1 - p) / n) * 2)


@pytest.mark.parametrize("R,L,V,B,n", [(4, 16, 2000, 64, 300), (5, 6, 777, 20, 200)])
def test_match_walk_trial_by_trial_against_oracle(R, L, V, B, n):
    """Target-sample matching on the table path (many trials) against the oracle's walk."""
    draft, trees, target = verification_case(R, L, V, B)
    alen, anode, nxt = host_outs(dt.accept_tree_match(oracle_to_device(trees, B), dev_bf16(target), 1.0, SEED, 0, n))
    bad = 0
    for r in range(R):
        rows = rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16")
        for t in range(n):
            ref = accept.walk_match(trees[r].parent, trees[r].token, trees[r].depth, rows, 1.0, SEED, t, r)
            bad += ref != (alen[t, r], anode[t, r], nxt[t, r])
    assert bad <= 2, bad   # draws within float rounding of a block or token boundary may differ


def test_match_walk_lazy_equals_tables():
    R, L, V, B = 6, 16, 4000, 64
    draft, trees, target = verification_case(R, L, V, B)
    dtree, tg = oracle_to_device(trees, B), dev_bf16(target)
    many = host_outs(dt.accept_tree_match(dtree, tg, 0.8, SEED, 0, 64))
    for t in (0, 5, 63):
        one = host_outs(dt.accept_tree_match(dtree, tg, 0.8, SEED, t, 1))
        for k in range(3):
            np.testing.assert_array_equal(one[k][0], many[k][t])


def test_match_walk_frequencies_within_3_sigma():
    """Stop-node frequencies over 10^6 trials per round against the oracle's exact law, and
    the emitted token's law at the most frequent stop node."""
    R, L, V, B = 4, 16, 3000, 64
    n = 1_000_000
    draft, trees, target = verification_case(R, L, V, B, seed=13)
    alen, anode, nxt = host_outs(dt.accept_tree_match(oracle_to_device(trees, B), dev_bf16(target), 1.0, SEED, 0, n))
    bins = beyond = 0
    for r in range(R):
        rows = rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16")
        stop, _, emit = accept.match_outcomes(trees[r].parent, trees[r].token, rows, 1.0)
        counts = np.bincount(anode[:, r], minlength=len(stop))
        for j, p in enumerate(stop):
            if p * n < 5:
                assert counts[j] <= max(10, 10 * p * n)
                continue
            bins += 1
            beyond += abs(counts[j] - n * p) > 3 * math.sqrt(n * p * (1 - p))
        j = int(np.argmax(stop))
        sel = nxt[anode[:, r] == j, r]
        m = sel.shape[0]
        for v in np.argsort(-emit[j])[:5]:
            f = emit[j][v]
            if f * m < 5:
                continue
            bins += 1
            beyond += abs(np.sum(sel == v) - m * f) > 3 * math.sqrt(m * f * (1 - f))
    assert beyond <= 0.01 * bins + 2, (beyond, bins)


def test_match_walk_full_vocabulary_sampled_rounds():
    """Verification config at full vocabulary (V = 151,936, B = 64): the one-trial walk
    (one workgroup per round) on three rounds, several trials, against the oracle."""
    R, L, V, B = 3, 16, 151936, 64
    draft, trees, target = verification_case(R, L, V, B)
    dtree, tg = oracle_to_device(trees, B), dev_bf16(target)
    rows = [rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16") for r in range(R)]
    bad = 0
    for t in range(4):
        alen, anode, nxt = host_outs(dt.accept_tree_match(dtree, tg, 1.0, SEED, t, 1))
        for r in range(R):
            ref = accept.walk_match(trees[r].parent, trees[r].token, trees[r].depth, rows[r], 1.0, SEED, t, r)
            bad += ref != (alen[0, r], anode[0, r], nxt[0, r])
    assert bad <= 1, bad


def test_match_walk_zero_temperature_is_greedy():
    R, L, V, B = 4, 16, 3000, 64
    draft, trees, target = verification_case(R, L, V, B)
    dtree, tg = oracle_to_device(trees, B), dev_bf16(target)
    g = host_outs(dt.accept_tree(dtree, tg, None, 0.0, SEED, 0, 2))
    m = host_outs(dt.accept_tree_match(dtree, tg, 0.0, SEED, 0, 2))
    for k in range(3):
        np.testing.assert_array_equal(g[k], m[k])
