"""GPU parity: marginal Top-B (a2 + a6) and TALON gated trees (a5 + a6) against the oracle."""
import numpy as np
import pytest
import torch

import draft_tree_construction_amd as dt
import synth
from oracle import gated, marginal, rowsweep
import oracle_pool as op
from parity_util import assert_tree_equal, dev_bf16, dev_f32, tree_to_host

pytestmark = pytest.mark.gpu


def oracle_marginal(z, K, B, beta):
    """Oracle tree plus its selection gap: score of the B-th minus the (B+1)-th prefix when
    they lie at different depths (inf otherwise)."""
    t = marginal.build_marginal(z, K, B, beta)
    L, V = z.shape
    Ke = min(B, V) if K == 0 else K
    lse = np.array([rowsweep.logsumexp_row(z[d]) for d in range(L)])
    ranks = np.stack([rowsweep.rank_order(z[d])[:Ke] for d in range(L)])
    zk = np.take_along_axis(z, ranks, axis=1)
    pops = marginal.heap_topb(zk, lse, B + 1, float(beta))
    # Within one depth the order is decided by exact logit sums on both sides; only a
    # boundary between two depths compares scores that carry each side's own LSE rounding.
    if len(pops) <= B or pops[B - 1]["depth"] == pops[B]["depth"]:
        return t, np.inf
    return t, pops[B - 1]["s"] - pops[B]["s"]


def check_marginal(host, dtype, K, B, beta, rounds=None):
    R = host.shape[0]
    d = dev_bf16(host) if dtype == "bf16" else dev_f32(host)
    tr = dt.build_tree_marginal(d, K, B, beta)
    h = tree_to_host(tr)
    exact = 0
    rounds = range(R) if rounds is None else rounds
    for r in rounds:
        z = rowsweep.as_f64(host[r], dtype)
        ref, gap = oracle_marginal(z, K, B, beta)
        exact += assert_tree_equal(h, r, ref, B, near_tie=gap <= 1e-5)
    return exact, len(list(rounds))


def test_marginal_tiny_config():
    """Tiny marginal config: R=4, L=4, V=32 fp32, K=B=8, beta=0."""
    exact, n = check_marginal(synth.tiny_marginal(), "f32", 8, 8, 0.0)
    assert exact == n


@pytest.mark.parametrize("R,L,V,K,B,beta", [
    (6, 16, 20000, 64, 64, 0.0),
    (5, 16, 3001, 0, 128, 0.0),     # K = min(B, V) = 128: DDTree's exact tree at B = 128
    (4, 7, 500, 16, 100, -0.3),
    (3, 3, 50, 50, 30, -2.0),
    (3, 1, 1000, 10, 10, 0.0),      # L = 1
    (2, 5, 40, 1, 5, 0.0),          # K = 1: argmax chain
    (2, 64, 700, 8, 128, -0.1),     # L = DTREE_MAX_L: 64 positions
])
def test_marginal_ddtree_shape_small(R, L, V, K, B, beta):
    host = synth.ddtree_logits(seed=20 + V, R=R, L=L, V=V)
    check_marginal(host, "bf16", K, B, beta)


def test_marginal_planted_ties():
    host = synth.tie_rows(300, 4 * 6, seed=3).reshape(4, 6, 300)
    exact, n = check_marginal(host, "bf16", 64, 64, 0.0)
    assert exact == n


def test_marginal_full_ddtree_config_all_rounds():
    """DDTree-shape config at full size (R=64, L=16, V=151936, K=B=64, beta=0) in one launch;
    every round checked node by node against the oracle (rounds whose Top-B cut is within
    1e-5 between two depths are checked for validity and shared scores, and counted)."""
    host = synth.ddtree_logits(seed=2)
    h = tree_to_host(dt.build_tree_marginal(dev_bf16(host), 64, 64, 0.0))
    ref = op.pmap(op.marginal_task, [(host[r], "bf16", 64, 64, 0.0) for r in range(64)])
    exact = sum(assert_tree_equal(h, r, t, 64, near_tie=gap <= 1e-5) for r, (t, gap) in enumerate(ref))
    near = sum(gap <= 1e-5 for _, gap in ref)
    assert exact == 64 - near and near <= 2, (exact, near)


def test_marginal_b128_full_vocabulary():
    """B = 128 with K = min(B, V) = 128 (DDTree's exact tree) on full-vocabulary rows, eight rounds."""
    host = synth.ddtree_logits(seed=2, R=8)
    h = tree_to_host(dt.build_tree_marginal(dev_bf16(host), 0, 128, -0.25))
    ref = op.pmap(op.marginal_task, [(host[r], "bf16", 0, 128, -0.25) for r in range(8)])
    exact = sum(assert_tree_equal(h, r, t, 128, near_tie=gap <= 1e-5) for r, (t, gap) in enumerate(ref))
    assert exact >= 7


def check_gated(host, K_root, mu, N, full_pool):
    R = host.shape[0]
    tr = dt.build_tree_gated(dev_bf16(host), K_root, mu, N)
    h = tree_to_host(tr)
    mu32 = float(np.float32(mu))
    for r in range(R):
        ref = gated.build_gated(rowsweep.as_f64(host[r], "bf16"), K_root, mu32, N, full_pool=full_pool)
        assert_tree_equal(h, r, ref, N)


@pytest.mark.parametrize("R,L,V,K_root,mu,N", [
    (6, 16, 300, 10, 0.03, 60),
    (4, 8, 120, 4, 0.2, 20),
    (4, 6, 64, 5, 1e-30, 40),
    (3, 10, 200, 3, 1.0, 50),
    (3, 16, 2000, 10, 0.03, 60),
    (2, 64, 400, 6, 0.05, 70),   # L = DTREE_MAX_L, N - K_root = DTREE_MAX_K
])
def test_gated_small(R, L, V, K_root, mu, N):
    host = synth.talon_logits(seed=40 + V, R=R, L=L, V=V)
    check_gated(host, K_root, mu, N, full_pool=True)


def test_gated_full_talon_config_all_rounds():
    """TALON config at full size (R=64, L=16, V=151936, K_root=10, mu=0.03, N=60): every round."""
    host = synth.talon_logits(seed=4)
    h = tree_to_host(dt.build_tree_gated(dev_bf16(host), 10, 0.03, 60))
    mu32 = float(np.float32(0.03))
    ref = op.pmap(op.gated_task, [(host[r], 10, mu32, 60) for r in range(64)])
    for r in range(64):
        assert_tree_equal(h, r, ref[r], 60)
