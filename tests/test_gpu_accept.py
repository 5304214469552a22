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
import oracle_pool as op
from parity_util import compare_with_margins, dev_bf16, dev_f32, full_verification_case, oracle_to_device

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


def test_greedy_walk_full_config_all_rounds():
    """Greedy walk on the full verification config: all 64 rounds against the oracle."""
    draft, trees, target = full_verification_case()
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, 64), dev_bf16(target), None, 0.0, SEED, 0, 2))
    ref = op.pmap(op.greedy_task, [(t.parent, t.token, t.depth, target[r, :t.n + 1]) for r, t in enumerate(trees)])
    for r in range(64):
        for t in range(2):
            assert (alen[t, r], anode[t, r], nxt[t, r]) == ref[r]


@pytest.mark.parametrize("R,L,V,B", [(8, 16, 5000, 64), (4, 5, 300, 20)])
def test_greedy_walk_matches_oracle(R, L, V, B):
    draft, trees, target = verification_case(R, L, V, B)
    dtree = oracle_to_device(trees, B)
    alen, anode, nxt = host_outs(dt.accept_tree(dtree, dev_bf16(target), None, 0.0, SEED, 0, 3))
    for r in range(R):
        ref = accept.walk_greedy(trees[r].parent, trees[r].token, trees[r].depth,
                                 rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16"))
        for t in range(3):
            assert (alen[t, r], anode[t, r], nxt[t, r]) == ref


def test_greedy_walk_one_workgroup_fallback():
    """600 rounds do not fit as four workgroups each, so the greedy walk runs one workgroup
    per round (the path every R up to the device's capacity / 4 skips); against the oracle."""
    R, L, V, B = 600, 4, 1000, 16
    draft = synth.ddtree_logits(seed=41, R=R, L=L, V=V)
    trees = [t for t, _ in op.pmap(op.marginal_task, [(draft[r], "bf16", 16, B, 0.0) for r in range(R)])]
    depth = np.stack([t.arrays(B)[2] for t in trees])
    target = synth.verification_target(draft, depth, seed=42)
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, B), dev_bf16(target), None, 0.0, SEED, 0, 1))
    for r in range(R):
        ref = accept.walk_greedy(trees[r].parent, trees[r].token, trees[r].depth,
                                 rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16"))
        assert (alen[0, r], anode[0, r], nxt[0, r]) == ref


@pytest.mark.parametrize("V", [1, 63, 200])
def test_greedy_walk_vocabulary_smaller_than_four_ranges(V):
    """V below four 64-token blocks leaves some of a round's four ranges empty."""
    R, L, B = 6, 3, 8
    draft = synth.ddtree_logits(seed=43 + V, R=R, L=L, V=V)
    trees = [marginal.build_marginal(rowsweep.as_f64(draft[r], "bf16"), min(B, V), B, 0.0) for r in range(R)]
    depth = np.stack([t.arrays(B)[2] for t in trees])
    target = synth.verification_target(draft, depth, seed=44)
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, B), dev_bf16(target), None, 0.0, SEED, 0, 2))
    for r in range(R):
        ref = accept.walk_greedy(trees[r].parent, trees[r].token, trees[r].depth,
                                 rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16"))
        for t in range(2):
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


def sampled_oracle(trees, target, draft, trials, T=1.0):
    """Per round: the oracle's walks for the given trial indices, with their margins, and
    the walk's exact stop law."""
    return op.pmap(op.sampled_task, [(t.parent, t.token, t.depth, target[r, :t.n + 1], draft[r], T, SEED, list(trials), r)
                                     for r, t in enumerate(trees)])


def test_sampled_walk_trial_by_trial_against_oracle():
    """Many trials per call (the table walk) against the oracle's walk under the shared Philox
    stream; a mismatch is allowed only where the oracle's decision margin is <= 1e-6."""
    R, L, V, B = 4, 16, 2000, 64
    draft, trees, target = verification_case(R, L, V, B)
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, B), dev_bf16(target), dev_bf16(draft),
                                                1.0, SEED, 0, 300))
    ref = sampled_oracle(trees, target, draft, range(300))
    bad = n = 0
    for r in range(R):
        b, k = compare_with_margins(zip(alen[:, r], anode[:, r], nxt[:, r]), ref[r][0])
        bad += b
        n += k
    assert bad <= n // 1000, (bad, n)


def test_sampled_walk_full_config_one_trial_against_oracle():
    """The verification config at full size (R = 64, 65 target rows, V = 151,936, B = 64,
    T = 1) with one trial per call -- four workgroups per round, the walk the benchmark
    times -- for trial indices 0..7, every round against the oracle's walk; a mismatch is
    allowed only where the oracle's decision margin is <= 1e-6, and at most 0.1 %."""
    draft, trees, target = full_verification_case()
    dtree, tg, dr = oracle_to_device(trees, 64), dev_bf16(target), dev_bf16(draft)
    trials = range(8)
    ref = sampled_oracle(trees, target, draft, trials)
    bad = n = 0
    for t in trials:
        alen, anode, nxt = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, t, 1))
        assert np.all(alen >= 0), "a round reported a failed walk"
        for r in range(64):
            b, k = compare_with_margins([(alen[0, r], anode[0, r], nxt[0, r])], [ref[r][0][t]])
            bad += b
            n += k
    assert n == 512 and bad <= n // 1000, (bad, n)


def test_narrow_walks_full_config_against_oracle():
    """accept_tree_narrow (one workgroup per round for every walk) on the full verification
    config: the greedy walk on all 64 rounds exactly, and the one-trial walk at T = 1 for trial
    indices 0..3 on every round, a mismatch allowed only where the oracle's decision margin is
    <= 1e-6 (at most 0.1 %)."""
    draft, trees, target = full_verification_case()
    dtree, tg, dr = oracle_to_device(trees, 64), dev_bf16(target), dev_bf16(draft)
    alen, anode, nxt = host_outs(dt.accept_tree_narrow(dtree, tg, None, 0.0, SEED, 0, 1))
    ref0 = op.pmap(op.greedy_task, [(t.parent, t.token, t.depth, target[r, :t.n + 1]) for r, t in enumerate(trees)])
    for r in range(64):
        assert (alen[0, r], anode[0, r], nxt[0, r]) == ref0[r]
    trials = range(4)
    ref = sampled_oracle(trees, target, draft, trials)
    bad = n = 0
    for t in trials:
        alen, anode, nxt = host_outs(dt.accept_tree_narrow(dtree, tg, dr, 1.0, SEED, t, 1))
        for r in range(64):
            b, k = compare_with_margins([(alen[0, r], anode[0, r], nxt[0, r])], [ref[r][0][t]])
            bad += b
            n += k
    assert n == 256 and bad <= n // 1000, (bad, n)


def test_narrow_and_default_walks_agree():
    """accept_tree_narrow and accept_tree on the same inputs: the greedy walks are identical;
    the one-trial walks at T = 1 agree but for decisions within float rounding (the two sum
    the LSE and the draw's block prefix in different orders): at most one of 48 differs."""
    R, L, V, B = 8, 16, 5000, 64
    draft, trees, target = verification_case(R, L, V, B)
    dtree, tg, dr = oracle_to_device(trees, B), dev_bf16(target), dev_bf16(draft)
    a = host_outs(dt.accept_tree(dtree, tg, None, 0.0, SEED, 0, 1))
    b = host_outs(dt.accept_tree_narrow(dtree, tg, None, 0.0, SEED, 0, 1))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    diff = 0
    for t in range(6):
        a = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, t, 1))
        b = host_outs(dt.accept_tree_narrow(dtree, tg, dr, 1.0, SEED, t, 1))
        diff += int(np.sum((a[0] != b[0]) | (a[1] != b[1]) | (a[2] != b[2])))
    assert diff <= 1, diff


MAX_ACCEPT_V = 262144  # DTREE_MAX_ACCEPT_V in include/dtree.h


def test_walks_at_the_largest_vocabulary():
    """accept_tree's envelope edge, V = 262,144 (the walk's dynamic LDS is largest there):
    the four-workgroup walks -- greedy, and T = 1 with one trial for trial indices 0..3 --
    against the oracle; a T = 1 mismatch only where the oracle's margin is <= 1e-6."""
    R, L, V, B = 3, 4, MAX_ACCEPT_V, 16
    draft, trees, target = verification_case(R, L, V, B)
    dtree, tg, dr = oracle_to_device(trees, B), dev_bf16(target), dev_bf16(draft)
    alen, anode, nxt = host_outs(dt.accept_tree(dtree, tg, None, 0.0, SEED, 0, 1))
    for r in range(R):
        ref = accept.walk_greedy(trees[r].parent, trees[r].token, trees[r].depth,
                                 rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16"))
        assert (alen[0, r], anode[0, r], nxt[0, r]) == ref
    trials = range(4)
    ref = sampled_oracle(trees, target, draft, trials)
    bad = n = 0
    for t in trials:
        alen, anode, nxt = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, t, 1))
        assert np.all(alen >= 0), "a round reported a failed walk"
        for r in range(R):
            b, k = compare_with_margins([(alen[0, r], anode[0, r], nxt[0, r])], [ref[r][0][t]])
            bad += b
            n += k
    assert n == R * len(trials) and bad <= 1, (bad, n)


def test_sampled_walk_full_vocab_frequencies():
    """Four rounds of the full-size verification config, 10^6 trials each (the table walk):
    stop-node frequencies within 3 sigma of the oracle's exact law, and the extra token's
    law at the most frequent stop node."""
    draft, trees, target = full_verification_case()
    R, n = 4, 1_000_000
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees[:R], 64), dev_bf16(target[:R]),
                                                dev_bf16(draft[:R]), 1.0, SEED, 0, n))
    bins = beyond = 0
    for r in range(R):
        t = trees[r]
        tab = accept.ResidualTables(t.parent, t.token, t.depth, rowsweep.as_f64(target[r, :t.n + 1], "bf16"),
                                    rowsweep.as_f64(draft[r], "bf16"), 1.0)
        stop, _ = accept.exact_outcomes(tab)
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
        f = tab.final[j]
        for v in np.argsort(-f)[:5]:
            if f[v] * m < 5:
                continue
            bins += 1
            beyond += abs(np.sum(sel == v) - m * f[v]) > 3 * math.sqrt(m * f[v] * (1 - f[v]))
    assert bins >= 8 and beyond <= 0.01 * bins + 2, (beyond, bins)


def test_sampled_walk_one_workgroup_fallback():
    """600 rounds need 2,400 workgroups of 1,024 threads at once, more than the device
    holds, so the one-trial walk runs one workgroup per round; against the oracle."""
    R, L, V, B = 600, 4, 1000, 16
    draft = synth.ddtree_logits(seed=31, R=R, L=L, V=V)
    trees = [t for t, _ in op.pmap(op.marginal_task, [(draft[r], "bf16", 16, B, 0.0) for r in range(R)])]
    depth = np.stack([t.arrays(B)[2] for t in trees])
    target = synth.verification_target(draft, depth, seed=32)
    dtree, tg, dr = oracle_to_device(trees, B), dev_bf16(target), dev_bf16(draft)
    trials = (0, 1, 2)
    ref = sampled_oracle(trees, target, draft, trials)
    bad = n = 0
    for t in trials:
        alen, anode, nxt = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, t, 1))
        for r in range(R):
            b, k = compare_with_margins([(alen[0, r], anode[0, r], nxt[0, r])], [ref[r][0][t]])
            bad += b
            n += k
    assert bad <= n // 1000 + 1, (bad, n)


def test_wait_bound_gives_documented_failure_outputs(monkeypatch):
    """With the cooperative walk's poll bound forced to 0 from the host, waits give up at
    once: each round ends with the documented -1 outputs or, where every partial was
    already there, the normal result; the call returns promptly. Without the bound the same
    call gives the normal results (the failure flags are cleared per call)."""
    R, L, V, B = 64, 16, 3000, 64
    draft, trees, target = verification_case(R, L, V, B, seed=14)
    dtree, tg, dr = oracle_to_device(trees, B), dev_bf16(target), dev_bf16(draft)
    good = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, 5, 1))
    monkeypatch.setenv("DTREE_ACCEPT_SPIN_LIMIT", "0")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    bad = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, 5, 1))
    e1.record()
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) < 100.0
    failed = 0
    for r in range(R):
        got = tuple(int(bad[k][0, r]) for k in range(3))
        if got == (-1, -1, -1):
            failed += 1
        else:
            assert got == tuple(int(good[k][0, r]) for k in range(3))
    assert failed >= 1
    monkeypatch.delenv("DTREE_ACCEPT_SPIN_LIMIT")
    again = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, 5, 1))
    for k in range(3):
        np.testing.assert_array_equal(again[k], good[k])


def _multichild_device(R):
    g = json.load(open(os.path.join(GOLD, "multichild_example.json")))
    from oracle.treeout import Tree
    tr = g["tree"]
    t = Tree()
    for i in range(1, len(tr["parent"])):
        t.add(tr["parent"][i], tr["token"][i], tr["depth"][i], -float(i))
    trees = [t] * R
    target = np.log(np.array(g["target_rows"], dtype=np.float64)).astype(np.float32)
    draft = np.log(np.array(g["draft_rows"], dtype=np.float64)).astype(np.float32)
    return g, trees, np.stack([target] * R), np.stack([draft] * R)


def test_multichild_example_frequencies_on_gpu():
    """The hand-worked multi-child example (a node with three children, one with two, two
    draft rows): stop frequencies over 10^6 trials against the hand fractions."""
    g, trees, target, draft = _multichild_device(2)
    n = 1_000_000
    alen, anode, nxt = host_outs(dt.accept_tree(oracle_to_device(trees, 5), dev_f32(target), dev_f32(draft), 1.0,
                                                SEED, 0, n))
    for r in range(2):
        for j, (a, b) in enumerate(g["stop"]):
            p = a / b
            f = np.mean(anode[:, r] == j)
            assert abs(f - p) <= 3 * math.sqrt(max(p * (1 - p), 1e-12) / n) + 1e-9, (r, j, f, p)
        # the root's final residual is (1, 0, 0, 0): every stop there emits token 0
        assert np.all(nxt[anode[:, r] == 0, r] == 0)
        at1 = nxt[anode[:, r] == 1, r]
        assert abs(np.mean(at1 == 3) - 12 / 13) <= 4 * math.sqrt((12 / 13) * (1 / 13) / max(at1.shape[0], 1))


def test_multichild_example_one_trial_against_oracle():
    """The same example through the one-trial walk (four workgroups per round; three of
    them hold no token of the four-token row), trial by trial against the oracle."""
    R = 8
    g, trees, target, draft = _multichild_device(R)
    dtree, tg, dr = oracle_to_device(trees, 5), dev_f32(target), dev_f32(draft)
    t0 = trees[0]
    tabs = [accept.ResidualTables(t0.parent, t0.token, t0.depth, target[r].astype(np.float64),
                                  draft[r].astype(np.float64), 1.0) for r in range(R)]
    bad = n = 0
    for t in range(64):
        alen, anode, nxt = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, t, 1))
        for r in range(R):
            b, k = compare_with_margins([(alen[0, r], anode[0, r], nxt[0, r])],
                                        [accept.walk_sampled_margin(tabs[r], t0.depth, SEED, t, r)])
            bad += b
            n += k
    assert bad <= 1, (bad, n)


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
    ref = op.pmap(op.match_task, [(t.parent, t.token, t.depth, target[r, :t.n + 1], 1.0, SEED, list(range(n)), r)
                                  for r, t in enumerate(trees)])
    bad = m = 0
    for r in range(R):
        b, k = compare_with_margins(zip(alen[:, r], anode[:, r], nxt[:, r]), ref[r])
        bad += b
        m += k
    assert bad <= m // 1000, (bad, m)   # only draws within 1e-6 of a boundary may differ


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
    ref = op.pmap(op.match_task, [(t.parent, t.token, t.depth, target[r, :t.n + 1], 1.0, SEED, list(range(4)), r)
                                  for r, t in enumerate(trees)])
    bad = 0
    for t in range(4):
        alen, anode, nxt = host_outs(dt.accept_tree_match(dtree, tg, 1.0, SEED, t, 1))
        for r in range(R):
            bad += compare_with_margins([(alen[0, r], anode[0, r], nxt[0, r])], [ref[r][t]])[0]
    assert bad <= 1, bad


def test_match_walk_zero_temperature_is_greedy():
    R, L, V, B = 4, 16, 3000, 64
    draft, trees, target = verification_case(R, L, V, B)
    dtree, tg = oracle_to_device(trees, B), dev_bf16(target)
    g = host_outs(dt.accept_tree(dtree, tg, None, 0.0, SEED, 0, 2))
    m = host_outs(dt.accept_tree_match(dtree, tg, 0.0, SEED, 0, 2))
    for k in range(3):
        np.testing.assert_array_equal(g[k], m[k])


def test_odd_vocabulary_last_token_on_aligned_rows():
    """Odd V (777): some rows start 16-byte aligned and take the vector loads, whose last
    unit straddles the row end. The largest target logit sits at the last index of every
    row, so the greedy walk must stop at the root and emit V - 1 in every round, and the
    matching and residual walks (one trial per call) must agree with the oracle."""
    R, L, V, B = 16, 6, 777, 20
    draft, trees, target = verification_case(R, L, V, B, seed=33)
    big = synth.bf16_from_f32(np.array([40.0], dtype=np.float32))[0]
    target = target.copy()
    target[:, :, V - 1] = big
    dtree, tg, dr = oracle_to_device(trees, B), dev_bf16(target), dev_bf16(draft)
    alen, anode, nxt = host_outs(dt.accept_tree(dtree, tg, None, 0.0, SEED, 0, 1))
    for r in range(R):
        want = accept.walk_greedy(trees[r].parent, trees[r].token, trees[r].depth,
                                  rowsweep.as_f64(target[r, :trees[r].n + 1], "bf16"))
        assert want[2] == V - 1 and (alen[0, r], anode[0, r], nxt[0, r]) == want
    ref_m = op.pmap(op.match_task, [(t.parent, t.token, t.depth, target[r, :t.n + 1], 1.0, SEED, [0, 1], r)
                                    for r, t in enumerate(trees)])
    ref_s = sampled_oracle(trees, target, draft, (0, 1))
    for t in (0, 1):
        m = host_outs(dt.accept_tree_match(dtree, tg, 1.0, SEED, t, 1))
        s = host_outs(dt.accept_tree(dtree, tg, dr, 1.0, SEED, t, 1))
        for r in range(R):
            assert compare_with_margins([(m[0][0, r], m[1][0, r], m[2][0, r])], [ref_m[r][t]])[0] == 0
            assert compare_with_margins([(s[0][0, r], s[1][0, r], s[2][0, r])], [ref_s[r][0][t]])[0] == 0
