"""Pins for the oracle's GRAFT edge scores, best-first builder and budget (CPU only)."""
import math

import numpy as np
import pytest

from oracle import marginal, tdes


def random_params(rng, V, L, hp=3, hc=4, hd=2, H=5, scale=1.0):
    return dict(Gp=rng.standard_normal((V, hp)), Gc=rng.standard_normal((V, hc)), Ed=rng.standard_normal((L, hd)),
                W=rng.standard_normal((H, hp + hc + hd)) * scale, b=rng.standard_normal(H) * scale,
                w=rng.standard_normal(H) * scale, b0=float(rng.standard_normal()))


def test_mlp_edge_by_hand():
    """One-wide embeddings, two hidden units: pre-activations (2.5, -1) -> ReLU (2.5, 0);
    f = 2 * 2.5 + 7 * 0 + 0.25. Swapping the parent and child tables, dropping the ReLU or
    the depth term changes the value."""
    prm = dict(Gp=np.array([[1.0], [0.0]]), Gc=np.array([[0.0], [2.0]]), Ed=np.array([[-1.0]]),
               W=np.array([[1.0, 1.0, 1.0], [1.0, -1.0, 0.0]]), b=np.array([0.5, 0.0]), w=np.array([2.0, 7.0]),
               b0=0.25)
    assert tdes.mlp_edge(0, 1, 1, prm) == 5.25
    # parent token 1, child token 0: pre = (0 + 0 - 1 + 0.5, 0 - 0) -> (0, 0): f = b0
    assert tdes.mlp_edge(1, 0, 1, prm) == 0.25


@pytest.mark.parametrize("seed", range(4))
def test_constant_edge_term_is_ddtree_with_a_depth_bonus(seed):
    """w = 0 makes f = b0 on every edge, so S_TDES(u) = sum of log q + s*b0*depth: the
    depth-bonus score with beta = s*b0 <= 0, under which a child never outscores its parent
    and best-first equals the marginal Top-B (the DDTree oracle, a separate heap)."""
    rng = np.random.default_rng(seed)
    L, V, K, B = 4, 40, 6, 20
    z = rng.standard_normal((L, V)) * 2.0
    prm = random_params(rng, V, L)
    prm["w"] = np.zeros_like(prm["w"])
    for beta in (0.0, -0.7):
        s = 0.5
        prm["b0"] = beta / s
        t, _ = tdes.build_tdes(z, 3, prm, K, B, s)
        ref = marginal.build_marginal(z, K, B, beta)
        got = dict(zip(t.paths(), t.score))
        want = dict(zip(ref.paths(), ref.score))
        assert set(got) == set(want)
        for p in got:
            assert abs(got[p] - want[p]) < 1e-9


def scan_best_first(z, root_tok, prm, K, B, s):
    """Best-first written without a heap: at every step scan every (taken node, child) pair
    not yet taken and take the best by (score, parent index, position among the parent's
    children sorted by edge score)."""
    L = z.shape[0]
    toks, rows = tdes.edge_rows(z, root_tok, prm, K, s)
    par, pci, dep, sc = [-1], [0], [0], [0.0]
    taken = set()
    while len(par) - 1 < B:
        best = None
        for n in range(len(par)):
            d = dep[n] + 1
            if d > L:
                continue
            S, order = rows[(d, pci[n])]
            for j, ci in enumerate(order):
                if (n, ci) in taken:
                    continue
                key = (-(sc[n] + S[ci]), n, j)
                if best is None or key < best[0]:
                    best = (key, n, ci)
        if best is None:
            break
        key, n, ci = best
        taken.add((n, ci))
        par.append(n)
        pci.append(ci)
        dep.append(dep[n] + 1)
        sc.append(-key[0])
    tok = [-1] + [toks[dep[i] - 1][pci[i]] for i in range(1, len(par))]
    return par, tok, dep, sc


@pytest.mark.parametrize("seed", range(5))
def test_heap_equals_frontier_scan_with_child_above_parent(seed):
    rng = np.random.default_rng(100 + seed)
    L, V, K, B = 4, 30, 5, 18
    z = rng.standard_normal((L, V)) * 1.5
    prm = random_params(rng, V, L, scale=1.5)
    s = 1.0
    t, gap = tdes.build_tdes(z, 7, prm, K, B, s)
    par, tok, dep, sc = scan_best_first(z, 7, prm, K, B, s)
    assert t.parent == par and t.token == tok and t.depth == dep
    np.testing.assert_allclose(t.score, sc, rtol=0, atol=1e-12)
    assert gap > 0


def test_positive_edges_make_children_outscore_parents():
    """With a large positive b0 every edge scores above zero, so each child outscores its
    parent and best-first runs depth first: a chain down to L, then the next branch."""
    rng = np.random.default_rng(7)
    L, V, K = 5, 30, 4
    z = rng.standard_normal((L, V))
    prm = random_params(rng, V, L)
    prm["w"] = np.zeros_like(prm["w"])
    prm["b0"] = 50.0
    t, _ = tdes.build_tdes(z, 0, prm, K, 8, 1.0)
    assert t.depth[1:6] == [1, 2, 3, 4, 5]
    assert t.parent[1:6] == [0, 1, 2, 3, 4]
    assert all(t.score[i] > t.score[t.parent[i]] for i in range(1, t.n + 1))
    # the chain takes each depth's best child (rank order at equal f)
    assert t.token[1] == int(np.argmax(z[0]))


def test_budget_larger_than_the_candidate_tree():
    rng = np.random.default_rng(8)
    L, V, K = 2, 10, 3
    z = rng.standard_normal((L, V))
    t, _ = tdes.build_tdes(z, 0, random_params(rng, V, L), K, 100, 0.3)
    assert t.n == K + K * K


@pytest.mark.parametrize("cv,cf", [(1.0, 10.0), (0.37, 20.0), (2.0, 3.0), (0.05, 7.9), (1.0, 0.0), (0.01, 500.0)])
def test_saba_budget_closed_form(cv, cf):
    """d/dB [B^beta / (B cv + cf)] = 0 at B* = beta cf / ((1 - beta) cv) (= cf / cv at
    beta = 1/2); the ratio rises before B* and falls after it, so the integer maximiser is
    floor(B*) or ceil(B*), clamped to [1, B_max]; a_t cancels."""
    B_max = 128
    for beta in (0.5, 0.3, 0.8):
        Bs = beta * cf / ((1 - beta) * cv)
        cands = sorted({min(max(int(math.floor(Bs)), 1), B_max), min(max(int(math.ceil(Bs)), 1), B_max)})
        u = lambda B: B ** beta / (B * cv + cf)
        want = max(cands, key=lambda B: (u(B), -B))
        for a in (1.0, 6.5):
            assert tdes.saba_budget(a, beta, cv, cf, B_max) == want
    assert tdes.saba_budget(1.0, 0.5, 1.0, 0.0, B_max) == 1
    assert tdes.saba_budget(1.0, 0.5, 0.01, 500.0, B_max) == B_max


def test_saba_bad_arguments():
    for args in [(0.0, 0.5, 1.0, 1.0, 8), (1.0, 1.0, 1.0, 1.0, 8), (1.0, 0.5, 0.0, 1.0, 8), (1.0, 0.5, 1.0, 1.0, 0)]:
        with pytest.raises(ValueError):
            tdes.saba_budget(*args)
