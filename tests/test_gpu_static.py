"""GPU parity: the static D x K grid expansion (TALON's fixed-shape baseline) against the oracle."""
import numpy as np
import pytest

import draft_tree_construction_amd as dt
import synth
from oracle import rowsweep, static
import oracle_pool as op
from parity_util import assert_tree_equal, dev_bf16, dev_f32, tree_to_host

pytestmark = pytest.mark.gpu


def check_static(host, dtype, K, D, rounds=None):
    R = host.shape[0]
    d = dev_bf16(host) if dtype == "bf16" else dev_f32(host)
    h = tree_to_host(dt.build_tree_static(d, K, D))
    for r in (range(R) if rounds is None else rounds):
        ref = static.build_static(rowsweep.as_f64(host[r], dtype), K, D)
        assert h["n"][r] == K * D
        assert_tree_equal(h, r, ref, K * D)


@pytest.mark.parametrize("R,L,V,K,D", [
    (6, 16, 300, 10, 6),     # TALON's comparison shape (60 nodes) on a small vocabulary
    (4, 8, 120, 4, 8),       # D = L
    (3, 6, 64, 64, 2),       # K = V = DTREE_MAX_K: 280 grid pairs, two ranking passes
    (3, 16, 2000, 16, 8),    # cap = DTREE_MAX_CAP
    (2, 5, 50, 1, 5),        # greedy chain
    (5, 3, 7000, 7, 1),      # one depth
    (1, 16, 151936, 10, 6),  # one round, full vocabulary
    (2, 64, 300, 2, 64),     # D = L = DTREE_MAX_L, K * D = DTREE_MAX_CAP
])
def test_static_small(R, L, V, K, D):
    host = synth.talon_logits(seed=60 + V, R=R, L=L, V=V)
    check_static(host, "bf16", K, D)


def test_static_f32():
    host = synth.tiny_marginal(seed=8, R=4, L=6, V=500)
    check_static(host, "f32", 12, 5)


def test_static_ties():
    """Logits from an 8-value grid: many paths tie; the order (parent slot, then token rank)
    is taken on the same float64 sums on both sides, so the trees match exactly."""
    R, L, V = 4, 6, 300
    host = synth.tie_rows(V, R * L, seed=13).reshape(R, L, V)
    check_static(host, "bf16", 10, 6)


def test_static_full_config_all_rounds():
    """Full size: R = 64 rounds, L = 16, V = 151,936 bf16, K = 10, D = 6 (60 nodes), every
    round against the oracle's literal K x V pool."""
    host = synth.talon_logits(seed=4)
    h = tree_to_host(dt.build_tree_static(dev_bf16(host), 10, 6))
    ref = op.pmap(op.static_task, [(host[r], 10, 6) for r in range(64)])
    for r in range(64):
        assert h["n"][r] == 60
        assert_tree_equal(h, r, ref[r], 60)
