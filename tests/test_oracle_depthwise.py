"""Pins for the oracle's DARTree depth-wise builder (CPU only).

The depth-wise super-tree is a heuristic with no closed form; it is pinned by
reductions: no correction -> the marginal tree; no pruning -> brute-force
best-first over corrected path scores (the exact "sequential correction with
heap" the DARTree summary names); width 1 -> the greedy corrected chain.
"""
import itertools
import math

import numpy as np
import pytest

import synth
from oracle import depthwise, marginal, rowsweep, treeout


def small_head(rng, V, dm, rank, L, scale):
    E = rng.standard_normal((V, dm)) * scale
    U = rng.standard_normal((L, dm, rank)) * scale
    P = rng.standard_normal((rank, V)) * scale
    return E, U, P


def lse(x):
    m = np.max(x)
    return m + math.log(np.sum(np.exp(x - m)))


def test_bf16_round_matches_generator_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 8, 20000)).astype(np.float32)
    x = np.concatenate([x, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)])
    ours = depthwise.bf16_round(x.astype(np.float64))
    gen = synth.f32_from_bf16(synth.bf16_from_f32(x)).astype(np.float64)
    np.testing.assert_array_equal(ours, gen)


@pytest.mark.parametrize("beta", [0.0, -0.4])
def test_zero_correction_equals_marginal_tree(beta):
    rng = np.random.default_rng(1)
    L, V, B = 4, 40, 12
    base = rng.standard_normal((L, V)) * 2.0
    E, U, P = small_head(rng, V, 16, 8, L, 0.3)
    U[:] = 0.0
    t = depthwise.build_depthwise(base, E, U, P, root_tok=5, K=B, W=B, B=B, beta=beta)
    m = marginal.build_marginal(base, B, B, beta)
    assert t.paths() == m.paths()
    np.testing.assert_allclose(t.score, m.score, atol=1e-12)


def corrected_brute_force(base, E, U, P, root_tok, K, B, beta):
    """Every prefix over C_1 x ... x C_L scored with its own path's correction, top-B by sort."""
    L, V = base.shape
    cands = [list(np.argsort(-base[d], kind="stable")[:K]) for d in range(L)]
    scored = []
    for d in range(1, L + 1):
        for ks in itertools.product(range(K), repeat=d):
            prev, s = root_tok, 0.0
            for i, k in enumerate(ks):
                h = depthwise.bf16_round(E[prev] @ U[i])
                z = base[i] + h @ P
                c = cands[i][k]
                s = min(s + (z[c] - lse(z)) + beta, s)
                prev = c
            scored.append((-s, d, tuple(cands[i][k] for i, k in enumerate(ks))))
    scored.sort()
    return {p: -ns for ns, _, p in scored[:B]}


@pytest.mark.parametrize("seed", [2, 3])
def test_no_pruning_equals_exact_corrected_best_first(seed):
    rng = np.random.default_rng(seed)
    L, V, K, B = 3, 20, 3, 9
    base = rng.standard_normal((L, V)) * 1.5
    E, U, P = small_head(rng, V, 8, 4, L, 0.8)
    t = depthwise.build_depthwise(base, E, U, P, root_tok=3, K=K, W=K ** (L - 1), B=B, beta=-0.1)
    ref = corrected_brute_force(base, E, U, P, 3, K, B, -0.1)
    got = {p: s for p, s in zip(t.paths()[1:], t.score[1:])}
    assert set(got) == set(ref)
    for p in got:
        assert abs(got[p] - ref[p]) < 1e-12
    treeout.check_invariants(t, B, L)


@pytest.mark.parametrize("seed", [5, 6])
def test_width_b_equals_exact_corrected_best_first(seed):
    """W = B already gives the exact best-first tree (the DARTree summary's sequential
    correction with a heap): a prefix in the global Top-B has fewer than B prefixes above
    it, so it is among the B best of its depth, whose parents are among the B best of theirs."""
    rng = np.random.default_rng(seed)
    L, V, K, B = 4, 24, 3, 10
    base = rng.standard_normal((L, V)) * 1.5
    E, U, P = small_head(rng, V, 8, 4, L, 0.8)
    t = depthwise.build_depthwise(base, E, U, P, root_tok=2, K=K, W=B, B=B, beta=0.0)
    ref = corrected_brute_force(base, E, U, P, 2, K, B, 0.0)
    got = {p: s for p, s in zip(t.paths()[1:], t.score[1:])}
    assert set(got) == set(ref)
    for p in got:
        assert abs(got[p] - ref[p]) < 1e-12


def test_width_one_is_greedy_corrected_chain():
    rng = np.random.default_rng(4)
    L, V, K = 5, 30, 4
    base = rng.standard_normal((L, V))
    E, U, P = small_head(rng, V, 8, 4, L, 0.8)
    t = depthwise.build_depthwise(base, E, U, P, root_tok=1, K=K, W=1, B=L, beta=0.0)
    prev, s = 1, 0.0
    for d in range(L):
        cands = np.argsort(-base[d], kind="stable")[:K]
        z = base[d] + depthwise.bf16_round(E[prev] @ U[d]) @ P
        sc = [s + (z[c] - lse(z)) for c in cands]
        best = int(np.argmax(sc))
        assert t.token[d + 1] == int(cands[best]) and t.parent[d + 1] == d
        s, prev = sc[best], int(cands[best])


def test_super_tree_invariants_workload_shape_small():
    R, L, V, dm, rank = 2, 6, 600, 32, 16
    base_b = synth.ddtree_logits(seed=2, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=3, R=R, L=L, V=V, d_model=dm, rank=rank)
    base = rowsweep.as_f64(base_b, "bf16")
    E64, U64, P64 = (synth.f32_from_bf16(a).astype(np.float64) for a in (E, U, P))
    for r in range(R):
        t, levels, gaps = depthwise.build_depthwise(base[r], E64, U64, P64, int(root[r]), K=8, W=32, B=40,
                                                    beta=-0.5, with_super=True)
        assert len(gaps) == L + 1 and all(g >= 0 for g in gaps)
        treeout.check_invariants(t, 40, L)
        assert len(levels[0]) == 8 and all(len(lv) <= 32 for lv in levels)
        for d in range(1, len(levels)):
            assert all(nd["ppos"] < len(levels[d - 1]) for nd in levels[d])


# ---- the sequential correction-with-heap builder (exact path-dependent best-first)

@pytest.mark.parametrize("seed,beta", [(7, 0.0), (8, -0.1), (9, -0.6)])
def test_sequential_equals_corrected_brute_force(seed, beta):
    """Popping one node at a time and correcting only that node gives the B best prefixes
    over every path scored with its own corrections (monotone scores, ancestors first)."""
    rng = np.random.default_rng(seed)
    L, V, K, B = 3, 20, 3, 11
    base = rng.standard_normal((L, V)) * 1.5
    E, U, P = small_head(rng, V, 8, 4, L, 0.8)
    t = depthwise.build_sequential(base, E, U, P, 4, K, B, beta)
    ref = corrected_brute_force(base, E, U, P, 4, K, B, beta)
    got = {p: s for p, s in zip(t.paths()[1:], t.score[1:])}
    assert set(got) == set(ref)
    for p in got:
        assert abs(got[p] - ref[p]) < 1e-12
    treeout.check_invariants(t, B, L)


@pytest.mark.parametrize("B", [1, 9, 40])
def test_sequential_equals_width_b_depthwise_node_for_node(B):
    """Same tree as the depth-wise builder at W = B, in the same canonical layout (pop order
    within a depth is S_d's order), on workload-shaped inputs with bf16 weights."""
    R, L, V, dm, rank = 3, 6, 500, 32, 16
    base_b = synth.ddtree_logits(seed=11, R=R, L=L, V=V)
    E, U, P, root = synth.correction_head(seed=12, R=R, L=L, V=V, d_model=dm, rank=rank)
    base = rowsweep.as_f64(base_b, "bf16")
    E64, U64, P64 = (synth.f32_from_bf16(a).astype(np.float64) for a in (E, U, P))
    for r in range(R):
        q = depthwise.build_sequential(base[r], E64, U64, P64, int(root[r]), 8, B, -0.2)
        t = depthwise.build_depthwise(base[r], E64, U64, P64, int(root[r]), K=8, W=B, B=B, beta=-0.2)
        assert (q.parent, q.token, q.depth) == (t.parent, t.token, t.depth)
        np.testing.assert_allclose(q.score, t.score, rtol=0, atol=1e-12)
        treeout.check_invariants(q, B, L)


def test_sequential_pops_in_score_order_and_reports_gaps():
    rng = np.random.default_rng(13)
    L, V, K, B = 5, 30, 4, 25
    base = rng.standard_normal((L, V))
    E, U, P = small_head(rng, V, 8, 4, L, 0.8)
    t, gaps = depthwise.build_sequential(base, E, U, P, 1, K, B, -0.3, with_gaps=True)
    assert t.n == B and len(gaps) == B and all(g >= 0 for g in gaps)
    # every node scores at most its parent, and no dropped prefix beats a kept one: the
    # last pop's gap is to the best prefix left out
    for i in range(1, len(t.parent)):
        assert t.score[i] <= t.score[t.parent[i]]
    assert np.isfinite(gaps[-1])


def test_sequential_chain_and_dry_heap():
    """K = 1: the heap holds one prefix at a time, so the tree is the corrected chain; a
    budget above the number of prefixes takes them all."""
    rng = np.random.default_rng(14)
    L, V = 4, 12
    base = rng.standard_normal((L, V))
    E, U, P = small_head(rng, V, 8, 4, L, 0.8)
    t = depthwise.build_sequential(base, E, U, P, 0, 1, 10, 0.0)
    assert t.n == L and t.parent == [-1, 0, 1, 2, 3]
    assert t.token[1:] == [int(np.argmax(base[d])) for d in range(L)]
    t2 = depthwise.build_sequential(base, E, U, P, 0, 2, 1000, -0.1)
    assert t2.n == 2 + 4 + 8 + 16
    with pytest.raises(ValueError):
        depthwise.build_sequential(base, E, U, P, 0, 2, 5, 0.1)
