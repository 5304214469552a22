"""Pins for the oracle's TALON gated tree (CPU only)."""
import math

import numpy as np
import pytest

import synth
from oracle import gated, rowsweep, treeout


def lse(x):
    m = np.max(x)
    return m + math.log(np.sum(np.exp(x - m)))


@pytest.mark.parametrize("seed", range(5))
def test_restricted_pool_equals_literal_full_pool(seed):
    """The literal pool P_d x V and the pool restricted to each position's top N-|T|
    tokens give the same tree (dominance: a token ranked below N-|T| always has N-|T|
    better siblings that pass the gate whenever it does)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((6, 80)) * 2.0
    for mu, N, kr in [(0.03, 20, 4), (0.2, 12, 3), (1e-4, 30, 5)]:
        a = gated.build_gated(z, kr, mu, N, full_pool=True)
        b = gated.build_gated(z, kr, mu, N, full_pool=False)
        assert a.paths() == b.paths() and a.parent == b.parent
        np.testing.assert_array_equal(a.score, b.score)


def test_mu_one_gives_root_layer_then_best_chain():
    rng = np.random.default_rng(9)
    L, V = 7, 50
    z = rng.standard_normal((L, V)) * 3.0
    t = gated.build_gated(z, 4, 1.0, 60)
    order0 = list(np.argsort(-z[0], kind="stable")[:4])
    assert t.token[1:5] == order0
    # then one node per depth: the best root-layer node extended by each position's argmax
    assert t.n == 4 + (L - 1)
    assert t.parent[5] == 1
    for d in range(1, L):
        assert t.token[4 + d] == int(np.argmax(z[d]))
        if d > 1:
            assert t.parent[4 + d] == 4 + d - 1


def test_tiny_mu_truncates_level_two_to_budget():
    rng = np.random.default_rng(10)
    L, V, N, kr = 5, 30, 25, 6
    z = rng.standard_normal((L, V))
    t = gated.build_gated(z, kr, 1e-30, N)
    assert t.n == N and max(t.depth) == 2
    # depth-2 nodes are the best N - kr pairs of (root-layer token, any token) by logit sum
    top = list(np.argsort(-z[0], kind="stable")[:kr])
    pairs = sorted(((-(z[0, a] + z[1, w]), i, w) for i, a in enumerate(top) for w in range(V)))
    want = {(top[i], w) for _, i, w in pairs[:N - kr]}
    got = {p for p in t.paths()[1:] if len(p) == 2}
    assert got == want


def test_invariants_talon_shape_small():
    b = synth.talon_logits(seed=4, R=3, L=16, V=4000)
    z = rowsweep.as_f64(b, "bf16")
    for r in range(3):
        t = gated.build_gated(z[r], 10, 0.03, 60, full_pool=False)
        treeout.check_invariants(t, 60, 16)
        assert t.token[1:11] == list(np.argsort(-z[r, 0], kind="stable")[:10])
        # every node below the root layer passes its depth's gate: p(u) >= mu * m_d
        paths = t.paths()
        by_depth = {}
        for i in range(1, t.n + 1):
            by_depth.setdefault(t.depth[i], []).append(i)
        for d in sorted(by_depth):
            if d == 1:
                continue
            parents = by_depth[d - 1]
            lp_next = z[r, d - 1] - lse(z[r, d - 1])
            anchor = max(t.score[p] for p in parents) + float(np.max(lp_next))
            for i in by_depth[d]:
                assert t.score[i] >= math.log(0.03) + anchor - 1e-9
        assert t.n <= 60


def test_argument_checks():
    z = np.zeros((3, 10))
    for kw in [dict(K_root=0, mu=0.1, N=5), dict(K_root=6, mu=0.1, N=5), dict(K_root=2, mu=0.0, N=5),
               dict(K_root=2, mu=1.5, N=5)]:
        with pytest.raises(ValueError):
            gated.build_gated(z, **kw)
